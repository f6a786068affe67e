"""GPU parity: every stage of the HIP path against the CPU oracle on the same
seeded inputs, through the C ABI (dsa_decode_amd.ops marshals arguments only).

Per stage, the inputs of both sides are identical: token inputs come from the
synthetic generators, and the inputs of later stages come from the oracle's
own earlier stages (never from a GPU result).  Bars:
  compress   one bf16 spacing (bf16 only) + 1e-5 * sum a|k|; bf16 >= 98% bit-equal
  scores     |g - o| <= 1e-3 |o| + 1e-5 A (A = forward-error scale), -inf exact
  top-k      bit-exact
  expand     bit-exact, every column written
  sparse MLA bf16: 2e-2 absolute; fp32: 1e-4 absolute; lse 2e-3 (bf16) / 1e-5 (fp32)
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from dsa_decode_amd import synth
from oracle import dsa_oracle as O
from tests.helpers import (act_from_f64, assert_compress_close, assert_scores_close,
                           assert_topk_property, dev, pool_cache_from_oracle, score_scale,
                           tile_pool_cache, untile_pool_cache)

pytestmark = pytest.mark.gpu


def ops():
    from dsa_decode_amd import ops as _ops
    return _ops


# ------------------------------------------------------------------ per-workload data
_CACHE: dict = {}


def wl_data(name: str) -> dict:
    """Synthetic inputs + the oracle's compress of them (cached per workload)."""
    if name in _CACHE:
        return _CACHE[name]
    wl = synth.workload(name)
    ti = synth.token_inputs(wl)
    comp = O.kpool_compress(ti["k"], ti["gate"], ti["valid"], ti["ape"], ti["seq_len"], wl.kp, wl.P_max)
    d = dict(wl=wl, ti=ti, comp=comp, ip=synth.index_params(wl))
    _CACHE[name] = d
    return d


def _absk_pool(d):
    ti, wl = d["ti"], d["wl"]
    return O.kpool_compress(ti["k"].abs(), ti["gate"], ti["valid"], ti["ape"], ti["seq_len"], wl.kp,
                            wl.P_max)["k_pool"]


def run_compress(d):
    ti, wl = d["ti"], d["wl"]
    return ops().dsa_kpool_compress(dev(ti["k"]), dev(ti["gate"]), dev(ti["valid"]), dev(ti["ape"]),
                                    dev(ti["seq_len"]), wl.kp, wl.P_max)


def check_compress(d):
    wl, comp = d["wl"], d["comp"]
    out = run_compress(d)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out["n_pools"].cpu().numpy(), comp["n_pools"])
    np.testing.assert_array_equal(out["first_valid"].cpu().numpy(), comp["first_valid"])
    np.testing.assert_array_equal(out["pool_start"].cpu().numpy(), comp["pool_start"])
    np.testing.assert_array_equal(out["pool_valid"].cpu().numpy().astype(bool), comp["pool_valid"])
    absk = _absk_pool(d)
    got = out["k_pool"].cpu()
    assert_compress_close(untile_pool_cache(got, wl.P_max), comp["k_pool"], absk, wl.torch_dtype)
    assert tuple(got.shape) == (wl.B, 16 * ((wl.P_max + 15) // 16), wl.D)


def scores_inputs(d, k_pool_override=None):
    wl = d["wl"]
    pc = pool_cache_from_oracle(d["comp"], wl.torch_dtype)
    if k_pool_override is not None:
        pc["k_pool"] = k_pool_override
    return pc


def run_scores(d, pc):
    ip, wl = d["ip"], d["wl"]
    return ops().dsa_index_scores(dev(ip["q"]), dev(ip["w"]), ip["scale"], dev(tile_pool_cache(pc["k_pool"])),
                                  dev(pc["pool_start"]), dev(pc["pool_valid"]), dev(ip["gamma"]),
                                  dev(ip["beta"]), ip["eps"], dev(ip["row_seq"]), dev(ip["row_pos"]),
                                  wl.kp)


def oracle_scores(d, pc, rows=None):
    ip, wl = d["ip"], d["wl"]
    return O.index_scores(ip["q"], ip["w"], ip["scale"], pc["k_pool"], pc["pool_start"], pc["pool_valid"],
                          ip["gamma"], ip["beta"], ip["eps"], ip["row_seq"], ip["row_pos"], wl.kp, rows=rows)


def check_scores(d, pc, rows=None):
    ip, wl = d["ip"], d["wl"]
    got = run_scores(d, pc).cpu().numpy()
    rows = list(range(wl.Q)) if rows is None else rows
    ref = oracle_scores(d, pc, rows)
    A = score_scale(ip["q"], ip["w"], ip["scale"], pc["k_pool"], ip["gamma"], ip["beta"], ip["eps"],
                    ip["row_seq"], rows)
    assert_scores_close(got[rows], ref, A)
    return ref


def check_topk(scores_np: np.ndarray, K: int):
    ref = O.topk_pools(scores_np, K)
    got = ops().dsa_topk_pools(dev(torch.from_numpy(scores_np)), K).cpu().numpy()
    np.testing.assert_array_equal(got, ref)
    return ref


def check_expand(ids: np.ndarray, row_seq, pool_start: np.ndarray, kp: int, W: int):
    ref = O.expand_selection(ids, row_seq, pool_start, kp, W)
    out = torch.full((ids.shape[0], W), 0x7fffffff, dtype=torch.int32, device="cuda")  # canary
    got = ops().dsa_expand_selection(dev(torch.from_numpy(ids.astype(np.int32))),
                                     dev(torch.as_tensor(np.asarray(row_seq, np.int32))),
                                     dev(torch.from_numpy(pool_start.astype(np.int32))), kp, W,
                                     token_ids=out).cpu().numpy()
    assert not (got == 0x7fffffff).any(), "unwritten slots in the token-id destination"
    np.testing.assert_array_equal(got, ref)
    return ref


def check_mla(q_lat, kv, row_seq, token_ids: np.ndarray, sm_scale, dtype, rows=None):
    out, lse = ops().dsa_sparse_mla_decode(dev(q_lat), dev(kv), dev(torch.as_tensor(np.asarray(row_seq, np.int32))),
                                           dev(torch.from_numpy(token_ids.astype(np.int32))), sm_scale)
    rows = list(range(q_lat.shape[0])) if rows is None else rows
    ref_o, ref_l = O.sparse_mla_decode(q_lat, kv, row_seq, token_ids, sm_scale, rows=rows)
    g = out.float().cpu().numpy()[rows]
    gl = lse.cpu().numpy()[rows]
    tol_o, tol_l = (2e-2, 2e-3) if dtype == torch.bfloat16 else (1e-4, 1e-5)
    err = np.abs(g - ref_o)
    assert err.max() <= tol_o, f"max out err {err.max()}"
    fin = np.isfinite(ref_l)
    assert (np.isfinite(gl) == fin).all()
    assert np.abs(gl[fin] - ref_l[fin]).max(initial=0) <= tol_l * np.maximum(1, np.abs(ref_l[fin])).max(initial=1)
    return g


# ------------------------------------------------------------------ tiny (fp32)
def test_tiny_compress():
    check_compress(wl_data("tiny"))


def test_tiny_scores_topk_expand_mla():
    d = wl_data("tiny")
    wl = d["wl"]
    pc = scores_inputs(d)
    ref_scores = check_scores(d, pc)
    ids = check_topk(ref_scores, wl.K)
    tok = check_expand(ids, d["ip"]["row_seq"].numpy(), d["comp"]["pool_start"], wl.kp, wl.W)
    mi = synth.mla_inputs(wl)
    check_mla(mi["q_lat"], mi["kv"], d["ip"]["row_seq"].numpy(), tok, mi["sm_scale"], wl.torch_dtype)


# ------------------------------------------------------------------ decode (bf16, 8192 ctx)
def test_decode_compress():
    check_compress(wl_data("decode"))


def test_decode_scores_topk_expand():
    d = wl_data("decode")
    wl = d["wl"]
    ref_scores = check_scores(d, scores_inputs(d))
    ids = check_topk(ref_scores, wl.K)
    check_expand(ids, d["ip"]["row_seq"].numpy(), d["comp"]["pool_start"], wl.kp, wl.W)


def test_decode_mla_on_selected_tokens():
    d = wl_data("decode")
    wl = d["wl"]
    ref_scores = oracle_scores(d, scores_inputs(d))
    ids = O.topk_pools(ref_scores, wl.K)
    tok = O.expand_selection(ids, d["ip"]["row_seq"].numpy(), d["comp"]["pool_start"], wl.kp, wl.W)
    mi = synth.mla_inputs(wl)
    check_mla(mi["q_lat"], mi["kv"], d["ip"]["row_seq"].numpy(), tok, mi["sm_scale"], wl.torch_dtype)


# ------------------------------------------------------------------ batched (32 ragged seqs)
def test_batched_compress():
    check_compress(wl_data("batched"))


def test_batched_scores_topk_expand_mla():
    d = wl_data("batched")
    wl = d["wl"]
    ref_scores = check_scores(d, scores_inputs(d))
    ids = check_topk(ref_scores, wl.K)
    rs = d["ip"]["row_seq"].numpy()
    tok = check_expand(ids, rs, d["comp"]["pool_start"], wl.kp, wl.W)
    mi = synth.mla_inputs(wl)
    check_mla(mi["q_lat"], mi["kv"], rs, tok, mi["sm_scale"], wl.torch_dtype, rows=list(range(0, 32, 3)))


# ------------------------------------------------------------------ long (4 x 262144, the bench workload)
def test_long_compress():
    check_compress(wl_data("long"))


def test_long_scores_topk_expand():
    d = wl_data("long")
    wl = d["wl"]
    ref_scores = check_scores(d, scores_inputs(d))
    ids = check_topk(ref_scores, wl.K)
    check_expand(ids, d["ip"]["row_seq"].numpy(), d["comp"]["pool_start"], wl.kp, wl.W)


def test_long_mla():
    d = wl_data("long")
    wl = d["wl"]
    rs = d["ip"]["row_seq"].numpy()
    tok = synth.random_token_ids(wl.Q, wl.W, wl.seq_len, rs.tolist(), seed=wl.seed)
    mi = synth.mla_inputs(wl)
    check_mla(mi["q_lat"], mi["kv"], rs, tok.numpy(), mi["sm_scale"], wl.torch_dtype)


# ------------------------------------------------------------------ prefill chunk (4096 rows, forced ties)
def test_prefill_scores_sampled_rows_and_topk():
    d = wl_data_prefill()
    wl = d["wl"]
    pc = scores_inputs(d, k_pool_override=synth.codebook_keys(wl))
    rows = [0, 1, 511, 2048, 3001, 4094, 4095]
    got = run_scores(d, pc)
    ref = oracle_scores(d, pc, rows)
    ip = d["ip"]
    A = score_scale(ip["q"], ip["w"], ip["scale"], pc["k_pool"], ip["gamma"], ip["beta"], ip["eps"],
                    ip["row_seq"], rows)
    g = got.cpu().numpy()
    assert_scores_close(g[rows], ref, A)
    # bit-exact top-k on the oracle's rows (ties straddle the cut there)
    check_topk(ref, wl.K)
    # the full-size selection on the GPU's own scores: every row valid
    ids = ops().dsa_topk_pools(got, wl.K).cpu().numpy()
    sample = list(range(0, 4096, 97)) + [4095]
    assert_topk_property(g[sample], ids[sample], wl.K)


def wl_data_prefill():
    # the prefill chunk pools a whole 131072-token sequence; the oracle's
    # compress is only needed for pool_start / pool_valid
    return wl_data("prefill")


def test_prefill_topk_forced_ties_full_size():
    s = synth.random_scores(4096, 32768, seed=77, tie_levels=300, neg_inf_frac=0.01, signed_zeros=True)
    got = ops().dsa_topk_pools(dev(s), 512).cpu().numpy()
    rows = list(range(0, 4096, 257)) + [4095]
    ref = O.topk_pools(s.numpy()[rows], 512)
    np.testing.assert_array_equal(got[rows], ref)


# ------------------------------------------------------------------ edge cases
@pytest.mark.parametrize("Q,P,K,ties", [(1, 1, 1, 0), (3, 7, 8, 0), (2, 1000, 8, 3), (4, 4097, 512, 50),
                                        (2, 65537, 512, 0), (4, 65536, 512, 40), (1, 65536, 2048, 0),
                                        (5, 300000, 64, 1000), (300, 5000, 100, 20), (4, 65536, 128, 30)])
def test_topk_shapes_ties_and_padding(Q, P, K, ties):
    s = synth.random_scores(Q, P, seed=Q * 1000 + P, tie_levels=ties, neg_inf_frac=0.3, signed_zeros=True)
    s[0, : P // 2] = -np.inf          # a row with few candidates
    if Q > 1:
        s[1, :] = -np.inf             # a row with none
    check_topk(s.numpy(), K)


def _shaped_score_rows(kind: str, Q: int, P: int, seed: int) -> np.ndarray:
    """fp32 score rows [Q, P] of a chosen shape along the pool index (each row
    shifted by its own offset): "rising" (a candidate list keeps growing),
    "falling", "equal" (one value per row: the order is the pool index alone),
    "random" (with ties, +-0, -inf holes, a short row and an empty row)."""
    rng = np.random.default_rng(seed)
    off = rng.standard_normal((Q, 1)).astype(np.float32)
    t = np.arange(P, dtype=np.float32)[None, :] / P
    if kind == "rising":
        s = off + t
    elif kind == "falling":
        s = off - t
    elif kind == "equal":
        s = np.broadcast_to(off, (Q, P)).copy()
    else:
        s = synth.random_scores(Q, P, seed=seed, tie_levels=64, neg_inf_frac=0.2, signed_zeros=True).numpy()
        s[0, : P - 100] = -np.inf      # a row with fewer candidates than K
        s[1, :] = -np.inf              # a row with none
    return np.ascontiguousarray(s, dtype=np.float32)


@pytest.mark.parametrize("kind,Q,P,K", [("rising", 512, 32768, 512), ("falling", 300, 20000, 100),
                                        ("equal", 256, 32768, 512), ("random", 260, 40000, 512),
                                        ("random", 300, 9000, 8), ("rising", 256, 16384, 1000),
                                        ("random", 256, 32768, 2048)])
def test_topk_shaped_rows_many_rows(kind, Q, P, K):
    # many rows (one workgroup per row, or chunk and merge launches for rows
    # over 32768) whose scores rise or fall along the pool index, tie
    # throughout, or are random with ties, +-0, holes, a short row and an
    # empty row: bit-exact against the oracle's top-k, with and without
    # expansion
    s = _shaped_score_rows(kind, Q, P, seed=Q + P + K)
    ref = O.topk_pools(s, K)
    sd = dev(torch.from_numpy(s))
    got = ops().dsa_topk_pools(sd, K)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), ref)
    kp, W = 4, 4 * K + 3
    ps = dev(torch.from_numpy((3 + kp * np.arange(P, dtype=np.int32))[None, :]))
    row_seq = dev(torch.zeros(Q, dtype=torch.int32))
    ids, tok = ops().dsa_topk_pools_expand(sd, K, row_seq, ps, kp, W)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ref)
    np.testing.assert_array_equal(tok.cpu().numpy(),
                                  O.expand_selection(ref, np.zeros(Q, np.int32), ps.cpu().numpy(), kp, W))


def test_topk_workspace_reuse_across_calls_and_shapes():
    # one zero-filled workspace for successive calls of different shapes: each
    # call must leave the counter block at the workspace's start at zero, or
    # the next call's merge would start from a wrong count
    shapes = [(4, 65536, 512), (2, 30000, 256), (3, 16384, 512), (4, 65536, 512)]
    need = max(ops().dsa_topk_workspace_bytes(Q, P, K) for Q, P, K in shapes)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")   # garbage, then the counter block zeroed
    ops().dsa_topk_workspace_init(ws)
    assert (ws[: ops().DSA_TOPK_COUNTER_BYTES] == 0).all() and (ws[ops().DSA_TOPK_COUNTER_BYTES:] == 0xA5).all()
    for i, (Q, P, K) in enumerate(shapes):
        s = synth.random_scores(Q, P, seed=90 + i, tie_levels=0 if i % 2 else 64, neg_inf_frac=0.1)
        got = ops().dsa_topk_pools(dev(s), K, workspace=ws).cpu().numpy()
        np.testing.assert_array_equal(got, O.topk_pools(s.numpy(), K))
        assert (ws[: ops().DSA_TOPK_COUNTER_BYTES] == 0).all()


@pytest.mark.parametrize("Q,P,K,kp,W,ties", [
    (4, 65536, 512, 4, 2048, 0),     # decode shape: split rows merged in one launch
    (3, 30000, 256, 4, 1100, 64),    # split rows, forced ties, padded width
    (2, 1000, 8, 3, 30, 0),          # one chunk per row
    (260, 33000, 64, 4, 256, 0),     # many rows: chunk launch + merge launch
])
def test_topk_pools_expand_matches_oracle(Q, P, K, kp, W, ties):
    # the fused entry point writes exactly what dsa_topk_pools then
    # dsa_expand_selection write: pool ids bit-exact with the oracle's top-k
    # and token ids bit-exact with the oracle's expansion of those ids, with
    # pools that do not exist, an invalid row, rows with fewer candidates
    # than K, and every token column written (canary fill)
    rng = np.random.default_rng(Q * 7 + P)
    s = synth.random_scores(Q, P, seed=Q + P + K, tie_levels=ties, neg_inf_frac=0.2).numpy()
    s[0, : P - K // 2] = -np.inf                    # row 0: fewer candidates than K
    B = 3
    pool_start = (np.arange(P, dtype=np.int64) * kp + rng.integers(0, 7, size=(B, 1))).astype(np.int32)
    pool_start[rng.random((B, P)) < 0.1] = -1       # pools that do not exist
    row_seq = rng.integers(0, B, size=Q).astype(np.int32)
    row_seq[Q - 1] = B                              # a row naming no sequence
    ref_ids = O.topk_pools(s, K)
    # the oracle expands rows of existing sequences; a row naming none gets
    # -1 throughout (the boundary turns the precondition violation into -1)
    ref_tok = O.expand_selection(ref_ids[:-1], row_seq[:-1], pool_start, kp, W)
    ref_tok = np.concatenate([ref_tok, np.full((1, W), -1, np.int32)])
    ids = torch.full((Q, K), 0x7fffffff, dtype=torch.int32, device="cuda")
    tok = torch.full((Q, W), 0x7fffffff, dtype=torch.int32, device="cuda")
    ops().dsa_topk_pools_expand(dev(torch.from_numpy(s)), K, dev(torch.from_numpy(row_seq)),
                                dev(torch.from_numpy(pool_start)), kp, W, pool_ids=ids, token_ids=tok)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    got = tok.cpu().numpy()
    assert not (got == 0x7fffffff).any(), "unwritten slots in the token-id destination"
    np.testing.assert_array_equal(got, ref_tok)


def test_topk_clustered_winners():
    # the merge of a split row first reads the head of each chunk's sorted
    # winner list; rows whose K winners crowd into one or a few chunks must
    # fall back to the full lists and still match
    Q, P, K = 5, 65536, 512
    rng = np.random.default_rng(11)
    s = np.empty((Q, P), np.float32)
    s[0] = np.arange(P, dtype=np.float32)                 # all winners in the last chunk
    s[1] = -np.arange(P, dtype=np.float32)                # all winners in the first chunk
    s[2] = rng.standard_normal(P).astype(np.float32)
    s[2, 4096:4096 + 300] += 10.0                         # 300 winners in one chunk, the rest spread
    s[3] = rng.standard_normal(P).astype(np.float32)
    s[3, ::4096] = 50.0                                   # one sure winner per chunk
    s[3, 8192:8192 + 200] = 20.0                          # 200 tied winners in one chunk
    s[4] = np.round(rng.standard_normal(P) * 4).astype(np.float32)  # coarse ties everywhere
    got = ops().dsa_topk_pools(dev(torch.from_numpy(s)), K).cpu().numpy()
    np.testing.assert_array_equal(got, O.topk_pools(s, K))


def test_topk_is_deterministic():
    s = dev(synth.random_scores(4, 65536, seed=5, tie_levels=100))
    a = ops().dsa_topk_pools(s, 512)
    b = ops().dsa_topk_pools(s, 512)
    assert torch.equal(a, b)


def test_compress_edge_cases():
    # holes, a fully invalid sequence, short sequences, kpool 1 / 3 / 8, fp32 and bf16
    for kp, dtype in [(1, torch.float32), (3, torch.bfloat16), (8, torch.bfloat16), (4, torch.float32)]:
        rng = np.random.default_rng(kp)
        B, T, D = 3, 70, 16
        k = torch.from_numpy(rng.standard_normal((B, T, D)).astype(np.float32)).to(dtype)
        gate = torch.from_numpy(rng.standard_normal((B, T, D)).astype(np.float32)).to(dtype)
        ape = torch.from_numpy((0.1 * rng.standard_normal((kp, D))).astype(np.float32))
        valid = np.ones((B, T), np.uint8)
        valid[0, :3] = 0
        valid[0, 20] = 0          # a hole
        valid[1, :] = 0           # nothing valid
        seq_len = np.array([70, 70, 33], np.int32)
        P_max = T // kp + 1
        comp = O.kpool_compress(k, gate, valid, ape, seq_len, kp, P_max)
        out = ops().dsa_kpool_compress(dev(k), dev(gate), dev(torch.from_numpy(valid)), dev(ape),
                                       dev(torch.from_numpy(seq_len)), kp, P_max)
        np.testing.assert_array_equal(out["n_pools"].cpu().numpy(), comp["n_pools"])
        np.testing.assert_array_equal(out["pool_start"].cpu().numpy(), comp["pool_start"])
        np.testing.assert_array_equal(out["pool_valid"].cpu().numpy().astype(bool), comp["pool_valid"])
        absk = O.kpool_compress(k.abs(), gate, valid, ape, seq_len, kp, P_max)["k_pool"]
        got = out["k_pool"].cpu()
        assert_compress_close(untile_pool_cache(got, P_max), comp["k_pool"], absk, dtype)
        # the layout's padding pools (past P_max, up to a whole 16-pool tile) are written as zeros
        full = untile_pool_cache(got, got.shape[1])
        assert (full[:, P_max:] == 0).all()


@pytest.mark.parametrize("H,D,dtype", [(16, 128, torch.bfloat16), (32, 128, torch.bfloat16),
                                       (8, 64, torch.bfloat16), (5, 32, torch.float32),
                                       (32, 128, torch.float32)])
def test_scores_paths_ragged_causal_and_mixed_rows(H, D, dtype):
    rng = np.random.default_rng(H * D)
    B, P, kp = 3, 1000, 4
    k_pool = torch.from_numpy(rng.standard_normal((B, P, D)).astype(np.float32)).to(dtype)
    pool_start = np.tile((np.arange(P) * kp + 2).astype(np.int32), (B, 1))
    pool_valid = (rng.random((B, P)) > 0.1).astype(np.uint8)
    pool_start[2, 700:] = -1
    pool_valid[2, 700:] = 0
    Q = 70                                   # several row batches, rows of all sequences mixed
    row_seq = rng.integers(0, B, Q).astype(np.int32)
    row_pos = rng.integers(0, P * kp + 10, Q).astype(np.int32)
    q = torch.from_numpy(rng.standard_normal((Q, H, D)).astype(np.float32)).to(dtype)
    w = torch.from_numpy((rng.random((Q, H)) / H).astype(np.float32))
    gamma = torch.from_numpy((1 + 0.02 * rng.standard_normal(D)).astype(np.float32))
    beta = torch.from_numpy((0.02 * rng.standard_normal(D)).astype(np.float32))
    got = ops().dsa_index_scores(dev(q), dev(w), D ** -0.5, dev(tile_pool_cache(k_pool)),
                                 dev(torch.from_numpy(pool_start)),
                                 dev(torch.from_numpy(pool_valid)), dev(gamma), dev(beta), 1e-5,
                                 dev(torch.from_numpy(row_seq)), dev(torch.from_numpy(row_pos)), kp).cpu().numpy()
    ref = O.index_scores(q, w, D ** -0.5, k_pool, pool_start, pool_valid, gamma, beta, 1e-5, row_seq, row_pos, kp)
    A = score_scale(q, w, D ** -0.5, k_pool, gamma, beta, 1e-5, row_seq, range(Q))
    assert_scores_close(got, ref, A)


@pytest.mark.parametrize("mu_over_sigma", [30.0, 100.0])
@pytest.mark.parametrize("Q", [4, 80])
def test_scores_offset_keys_layernorm(mu_over_sigma, Q):
    # The score kernels fold the LayerNorm into the contraction and take its
    # statistics from sum x and sum x^2; pooled keys with a large common mean
    # are where that loses precision.  k_norm subtracts the mean ("Module
    # glm5next_dsa", "Traps carried from Slice 8"), so these keys must score
    # as zero-mean ones do.  Keys: mu + sigma * N(0, 1) per channel, with a
    # per-pool sign on mu; Q = 4 takes the decode kernel, Q = 80 the many-rows
    # kernel.  The header states |mean| <= 100 sigma as the supported domain.
    rng = np.random.default_rng(int(mu_over_sigma) * 7 + Q)
    B, P, kp, H, D = 2, 3000, 4, 32, 128
    sigma = 0.05
    sign = np.where(rng.random((B, P, 1)) < 0.5, -1.0, 1.0)
    x = sign * mu_over_sigma * sigma + sigma * rng.standard_normal((B, P, D))
    k_pool = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    ps = np.tile((np.arange(P) * kp + 1).astype(np.int32), (B, 1))
    pv = np.ones((B, P), np.uint8)
    row_seq = (np.arange(Q) % B).astype(np.int32)
    row_pos = np.full(Q, P * kp + 3, np.int32)
    row_pos[1::3] = rng.integers(kp, P * kp, row_pos[1::3].size)  # causal cut inside the row too
    q = torch.from_numpy(rng.standard_normal((Q, H, D)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.random((Q, H)) / H).astype(np.float32))
    gamma = torch.from_numpy((1 + 0.02 * rng.standard_normal(D)).astype(np.float32))
    beta = torch.from_numpy((0.02 * rng.standard_normal(D)).astype(np.float32))
    got = ops().dsa_index_scores(dev(q), dev(w), D ** -0.5, dev(tile_pool_cache(k_pool)),
                                 dev(torch.from_numpy(ps)), dev(torch.from_numpy(pv)), dev(gamma), dev(beta), 1e-5,
                                 dev(torch.from_numpy(row_seq)), dev(torch.from_numpy(row_pos)), kp).cpu().numpy()
    ref = O.index_scores(q, w, D ** -0.5, k_pool, ps, pv, gamma, beta, 1e-5, row_seq, row_pos, kp)
    A = score_scale(q, w, D ** -0.5, k_pool, gamma, beta, 1e-5, row_seq, range(Q))
    assert np.isfinite(ref).sum() > Q * P // 3
    assert_scores_close(got, ref, A)


def test_scores_duplicate_pools_are_bit_identical():
    d = wl_data("prefill")
    wl = d["wl"]
    pc = scores_inputs(d, k_pool_override=synth.codebook_keys(wl, n_codes=4))
    got = run_scores(d, pc).cpu().numpy()
    kp_rows = pc["k_pool"][0].view(torch.int16).numpy()
    _, code = np.unique(kp_rows, axis=0, return_inverse=True)
    for r in (0, 4095):
        s = got[r]
        for c in range(4):
            vals = s[(code.ravel() == c) & np.isfinite(s)]
            assert np.unique(vals).size == 1


@pytest.mark.parametrize("Hm,Dl,dtype,W", [(64, 512, torch.bfloat16, 2048), (16, 512, torch.bfloat16, 70),
                                           (32, 512, torch.bfloat16, 1), (4, 64, torch.bfloat16, 100),
                                           (4, 64, torch.float32, 300), (128, 512, torch.bfloat16, 300)])
def test_mla_shapes_holes_and_empty_rows(Hm, Dl, dtype, W):
    rng = np.random.default_rng(Hm + Dl + W)
    B, T, Q = 2, 5000, 3
    q_lat = torch.from_numpy(rng.standard_normal((Q, Hm, Dl)).astype(np.float32)).to(dtype)
    kv = torch.from_numpy(rng.standard_normal((B, T, Dl)).astype(np.float32)).to(dtype)
    row_seq = np.array([1, 0, 1], np.int32)
    tok = synth.random_token_ids(Q, W, [T, T], row_seq.tolist(), seed=W, hole_frac=0.2).numpy()
    tok[2, :] = -1                       # a row with nothing selected
    check_mla(q_lat, kv, row_seq, tok, Dl ** -0.5, dtype)


@pytest.mark.parametrize("W", [1000, 5000, 16384])
def test_mla_split_merge_levels(W):
    # 16, 79 and 256 id slices per row, up to the largest W the entry point
    # accepts: the merge of the slices' partials in batches with a running
    # maximum
    rng = np.random.default_rng(W)
    B, T, Q, Hm = 2, 20000, 2, 64
    q_lat = torch.from_numpy(rng.standard_normal((Q, Hm, 512)).astype(np.float32)).to(torch.bfloat16)
    kv = torch.from_numpy(rng.standard_normal((B, T, 512)).astype(np.float32)).to(torch.bfloat16)
    row_seq = np.array([1, 0], np.int32)
    tok = synth.random_token_ids(Q, W, [T, T], row_seq.tolist(), seed=W, hole_frac=0.1).numpy()
    check_mla(q_lat, kv, row_seq, tok, 512 ** -0.5, torch.bfloat16)


def _distinct_ids_below(rng, Q, W, limits, hole_frac=0.0):
    """Per row q, W distinct random token ids in [0, limits[q]) (fewer when the
    range is smaller; the rest -1), with a fraction turned into -1 holes."""
    out = np.full((Q, W), -1, np.int32)
    for qi in range(Q):
        n = int(limits[qi])
        take = min(W, n)
        if take == n:
            ids = rng.permutation(n)
        else:
            ids = np.unique(rng.integers(0, n, size=2 * take + 64))
            while ids.size < take:
                ids = np.unique(np.concatenate([ids, rng.integers(0, n, size=take)]))
            ids = rng.permutation(ids)[:take]
        out[qi, :take] = ids
    if hole_frac > 0:
        out[rng.random(out.shape) < hole_frac] = -1
    return out


@pytest.mark.parametrize("Q,Hm,W", [(256, 64, 1000), (1024, 16, 130), (300, 64, 2048), (1030, 16, 200),
                                    (600, 32, 333),
                                    # 64 heads: three 32-id blocks (the last holding one id), three
                                    # full ones, the largest list the pipelined kernel takes, and one
                                    # id more (the eight-wave kernel)
                                    (256, 64, 65), (256, 64, 96), (256, 64, 4096), (256, 64, 4097)])
def test_mla_many_rows_path(Q, Hm, W):
    # enough (row, head group) pairs that each workgroup runs over all of its
    # row's ids with the online softmax (no split partials): ragged last
    # blocks, holes, empty rows, rows whose first blocks are all holes, and a
    # row count that is not a multiple of 8
    rng = np.random.default_rng(Q + W)
    B, T = 3, 6000
    q_lat = torch.from_numpy(rng.standard_normal((Q, Hm, 512)).astype(np.float32)).to(torch.bfloat16)
    kv = torch.from_numpy(rng.standard_normal((B, T, 512)).astype(np.float32)).to(torch.bfloat16)
    row_seq = (np.arange(Q) % B).astype(np.int32)
    tok = _distinct_ids_below(rng, Q, W, np.full(Q, T), hole_frac=0.15)
    tok[5, :] = -1                          # nothing selected
    tok[7, : min(W, 200)] = -1              # the first blocks empty, later ones not
    tok[9, 1:] = -1                         # a single token
    rows = sorted({0, 5, 7, 9, Q - 1} | set(rng.choice(Q, 12, replace=False).tolist()))
    lib = ops()._lib.load()
    assert lib.dsa_sparse_mla_workspace_bytes(Q, Hm, 512, W, 1) == 0   # no split partials
    check_mla(q_lat, kv, row_seq, tok, 512 ** -0.5, torch.bfloat16, rows=rows)


def test_mla_prefill_chunk_full_size_sampled_rows():
    # the prefill chunk's shape: 4096 rows at positions 126976 .. 131071 of one
    # 131072-token sequence, 2048 ids per row (causal: ids at or before the
    # row's position), 64 heads over the 512 latent; sampled rows against the
    # oracle, every row finite and lse finite
    wl = synth.workload("prefill")
    rng = np.random.default_rng(4096)
    mi = synth.mla_inputs(wl)
    ip = synth.index_params(wl)
    pos = ip["row_pos"].numpy()
    tok = _distinct_ids_below(rng, wl.Q, wl.W, pos + 1)
    rows = [0, 1, 777, 2048, 4095] + rng.choice(wl.Q, 5, replace=False).tolist()
    g = check_mla(mi["q_lat"], mi["kv"], ip["row_seq"].numpy(), tok, mi["sm_scale"], torch.bfloat16, rows=rows)
    assert np.isfinite(g).all()


def test_mla_one_dominant_token_per_row():
    # every head of row r puts its softmax mass on one token, in a different id
    # slice per row: the merge weights of the slices must carry it
    # (q is aligned with that token's row, so the outputs keep the magnitude of
    # a kv row and the bf16 bound still applies)
    rng = np.random.default_rng(5)
    B, T, Q, Hm, W = 1, 8192, 4, 32, 2048
    kv = rng.standard_normal((B, T, 512)).astype(np.float32)
    q = 0.1 * rng.standard_normal((Q, Hm, 512)).astype(np.float32)
    tok = synth.random_token_ids(Q, W, [T], [0] * Q, seed=77).numpy()
    for r, c in enumerate([0, 700, 1337, W - 1]):
        row = kv[0, tok[r, c]]
        q[r] += 40.0 * np.sqrt(512) * row / (row @ row)   # logit of that token: 40
    o = check_mla(torch.from_numpy(q).to(torch.bfloat16), torch.from_numpy(kv).to(torch.bfloat16), [0] * Q, tok,
                  512 ** -0.5, torch.bfloat16)
    for r, c in enumerate([0, 700, 1337, W - 1]):
        assert np.abs(o[r] - kv[0, tok[r, c]][None, :]).max() <= 2e-2


def test_mla_workspace_reuse_across_calls_and_shapes():
    # one workspace for successive calls of different shapes: partials of one
    # call must not leak into the next; outputs start as NaN so that a merge
    # that never ran shows
    shapes = [(4, 64, 2048), (2, 128, 5000), (3, 16, 300), (4, 64, 2048), (1, 64, 16384), (130, 32, 200)]
    need = max(ops().dsa_sparse_mla_workspace_bytes(Q, Hm, 512, W, ops().DSA_BF16) for Q, Hm, W in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    B, T = 2, 20000
    for i, (Q, Hm, W) in enumerate(shapes):
        rng = np.random.default_rng(40 + i)
        q_lat = torch.from_numpy(rng.standard_normal((Q, Hm, 512)).astype(np.float32)).to(torch.bfloat16)
        kv = torch.from_numpy(rng.standard_normal((B, T, 512)).astype(np.float32)).to(torch.bfloat16)
        row_seq = (np.arange(Q) % B).astype(np.int32)
        tok = synth.random_token_ids(Q, W, [T, T], row_seq.tolist(), seed=i, hole_frac=0.1).numpy()
        out = torch.full((Q, Hm, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        o, lse = ops().dsa_sparse_mla_decode(dev(q_lat), dev(kv), dev(torch.from_numpy(row_seq)),
                                             dev(torch.from_numpy(tok)), 512 ** -0.5, out=out, workspace=ws)
        ref_o, ref_l = O.sparse_mla_decode(q_lat, kv, row_seq, tok, 512 ** -0.5)
        g = o.float().cpu().numpy()
        assert np.isfinite(g).all()
        assert np.abs(g - ref_o).max() <= 2e-2
        assert np.abs(lse.cpu().numpy() - ref_l).max() <= 2e-3 * np.abs(ref_l).max()


def test_mla_permutation_invariant():
    rng = np.random.default_rng(9)
    q_lat = torch.from_numpy(rng.standard_normal((1, 64, 512)).astype(np.float32)).to(torch.bfloat16)
    kv = torch.from_numpy(rng.standard_normal((1, 4096, 512)).astype(np.float32)).to(torch.bfloat16)
    tok = synth.random_token_ids(1, 2048, [4096], [0], seed=3).numpy()
    a = check_mla(q_lat, kv, [0], tok, 512 ** -0.5, torch.bfloat16)
    b = check_mla(q_lat, kv, [0], tok[:, ::-1].copy(), 512 ** -0.5, torch.bfloat16)
    assert np.abs(a - b).max() <= 2e-2


def test_end_to_end_decode_pipeline_on_gpu():
    """All stages chained on the GPU (compress -> scores -> top-k -> expand -> MLA)
    for the decode workload, against the oracle's own pipeline on the same
    token inputs.  Selection: every pool the oracle ranks clearly inside the cut
    (beyond the score tolerance) is selected by the GPU, and every GPU pick
    scores no lower than the oracle's K-th score minus that tolerance.  When
    the two selections are the same set (the usual case) the attention outputs
    must agree (attention is invariant to the order of the ids)."""
    d = wl_data("decode")
    wl, ip = d["wl"], d["ip"]
    comp = run_compress(d)
    scores = ops().dsa_index_scores(dev(ip["q"]), dev(ip["w"]), ip["scale"], comp["k_pool"], comp["pool_start"],
                                    comp["pool_valid"], dev(ip["gamma"]), dev(ip["beta"]), ip["eps"],
                                    dev(ip["row_seq"]), dev(ip["row_pos"]), wl.kp)
    ids = ops().dsa_topk_pools(scores, wl.K)
    tok = ops().dsa_expand_selection(ids, dev(ip["row_seq"]), comp["pool_start"], wl.kp, wl.W)
    mi = synth.mla_inputs(wl)
    out, _ = ops().dsa_sparse_mla_decode(dev(mi["q_lat"]), dev(mi["kv"]), dev(ip["row_seq"]), tok, mi["sm_scale"])
    torch.cuda.synchronize()
    # the oracle's pipeline from the same token inputs
    pc = pool_cache_from_oracle(d["comp"], wl.torch_dtype)
    ref = oracle_scores(d, pc)
    ref_ids = O.topk_pools(ref, wl.K)
    ref_tok = O.expand_selection(ref_ids, ip["row_seq"].numpy(), d["comp"]["pool_start"], wl.kp, wl.W)
    ref_o, _ = O.sparse_mla_decode(mi["q_lat"], mi["kv"], ip["row_seq"], ref_tok, mi["sm_scale"])
    s = ref[0]
    kth = np.sort(s[np.isfinite(s)])[::-1][wl.K - 1]
    tol = 1e-3 * abs(kth) + 1e-4
    sel = ids.cpu().numpy()[0]
    assert (sel >= 0).all() and len(set(sel.tolist())) == wl.K
    assert (s[sel] >= kth - tol).all()
    clearly_in = np.flatnonzero(s > kth + tol)
    assert set(clearly_in.tolist()) <= set(sel.tolist())
    if set(sel.tolist()) == set(ref_ids[0].tolist()):
        assert np.abs(out.float().cpu().numpy() - ref_o).max() <= 2e-2


def test_end_to_end_batched_pipeline_on_gpu():
    """The batched decode workload (32 sequences of ragged lengths with left
    padding) through the whole GPU pipeline (compress -> scores -> top-k +
    expand -> sparse MLA), against the oracle's own pipeline on the same token
    inputs, row by row: every pool the oracle ranks clearly inside the cut is
    selected, every GPU pick scores no lower than the oracle's K-th score minus
    the tolerance, every token id lies in [first valid, length) of its own
    sequence, and rows whose selection equals the oracle's agree in attention."""
    d = wl_data("batched")
    wl, ip = d["wl"], d["ip"]
    comp = run_compress(d)
    scores = ops().dsa_index_scores(dev(ip["q"]), dev(ip["w"]), ip["scale"], comp["k_pool"], comp["pool_start"],
                                    comp["pool_valid"], dev(ip["gamma"]), dev(ip["beta"]), ip["eps"],
                                    dev(ip["row_seq"]), dev(ip["row_pos"]), wl.kp)
    ids, tok = ops().dsa_topk_pools_expand(scores, wl.K, dev(ip["row_seq"]), comp["pool_start"], wl.kp, wl.W)
    mi = synth.mla_inputs(wl)
    out, _ = ops().dsa_sparse_mla_decode(dev(mi["q_lat"]), dev(mi["kv"]), dev(ip["row_seq"]), tok, mi["sm_scale"])
    torch.cuda.synchronize()
    ids, tok, out = ids.cpu().numpy(), tok.cpu().numpy(), out.float().cpu().numpy()
    rows = [0, 7, 13, 31]
    pc = pool_cache_from_oracle(d["comp"], wl.torch_dtype)
    ref = oracle_scores(d, pc, rows)
    first = d["comp"]["first_valid"]
    same = []
    for i, r in enumerate(rows):
        s = ref[i]
        fin = np.sort(s[np.isfinite(s)])[::-1]
        kth = fin[wl.K - 1]
        tol = 1e-3 * abs(kth) + 1e-4
        sel = ids[r]
        assert (sel >= 0).all() and len(set(sel.tolist())) == wl.K
        assert (s[sel] >= kth - tol).all()
        assert set(np.flatnonzero(s > kth + tol).tolist()) <= set(sel.tolist())
        b = int(ip["row_seq"][r])
        t = tok[r]
        assert (t >= first[b]).all() and (t < wl.seq_len[b]).all() and len(set(t.tolist())) == wl.W
        if set(sel.tolist()) == set(O.topk_pools(s[None], wl.K)[0].tolist()):
            same.append((i, r))
    assert same, "no row selected the oracle's set"
    ref_tok = np.stack([tok[r] for _, r in same])
    ro, _ = O.sparse_mla_decode(mi["q_lat"][[r for _, r in same]], mi["kv"], ip["row_seq"][[r for _, r in same]],
                                ref_tok, mi["sm_scale"])
    assert np.abs(out[[r for _, r in same]] - ro).max() <= 2e-2


def test_end_to_end_prefill_chunk_on_gpu():
    """The prefill chunk chained on the GPU (scores over the forced-ties pool
    cache -> top-k + expand -> sparse MLA over the selected tokens), checked on
    sampled rows against the oracle: the selection is valid for the oracle's
    scores (clearly-in pools selected, no pick below the K-th score minus the
    tolerance; ties at the cut may resolve either way within tolerance), token
    ids are causal and distinct, and the attention over the GPU's own token ids
    matches the oracle's attention over the same ids."""
    d = wl_data_prefill()
    wl, ip = d["wl"], d["ip"]
    pc = scores_inputs(d, k_pool_override=synth.codebook_keys(wl))
    scores = run_scores(d, pc)
    ids, tok = ops().dsa_topk_pools_expand(scores, wl.K, dev(ip["row_seq"]), dev(pc["pool_start"]), wl.kp, wl.W)
    mi = synth.mla_inputs(wl)
    out, lse = ops().dsa_sparse_mla_decode(dev(mi["q_lat"]), dev(mi["kv"]), dev(ip["row_seq"]), tok,
                                           mi["sm_scale"])
    torch.cuda.synchronize()
    ids, tok = ids.cpu().numpy(), tok.cpu().numpy()
    rows = [0, 1234, 4095]
    ref = oracle_scores(d, pc, rows)
    A = score_scale(ip["q"], ip["w"], ip["scale"], pc["k_pool"], ip["gamma"], ip["beta"], ip["eps"],
                    ip["row_seq"], rows)
    for i, r in enumerate(rows):
        s = ref[i]
        kth = np.sort(s[np.isfinite(s)])[::-1][wl.K - 1]
        tol = 1e-3 * abs(kth) + 1e-5 * A[i][np.isfinite(s)].max()
        sel = ids[r]
        assert (sel >= 0).all() and len(set(sel.tolist())) == wl.K
        assert (s[sel] >= kth - tol).all()
        assert set(np.flatnonzero(s > kth + tol).tolist()) <= set(sel.tolist())
        t = tok[r]
        assert (t >= 0).all() and (t <= int(ip["row_pos"][r])).all() and len(set(t.tolist())) == wl.W
    ro, rl = O.sparse_mla_decode(mi["q_lat"], mi["kv"], ip["row_seq"], tok, mi["sm_scale"], rows=rows)
    assert np.abs(out.float().cpu().numpy()[rows] - ro).max() <= 2e-2
    assert np.abs(lse.cpu().numpy()[rows] - rl).max() <= 2e-3 * max(1.0, np.abs(rl).max())


def _streamed_vs_oracle(scores: np.ndarray, ids: np.ndarray, tok: np.ndarray, rows, row_seq, pool_start,
                        kp: int, K: int, W: int) -> None:
    """The streamed entry's pool ids and token ids on the given rows against
    the oracle's top-k and expansion of the same score rows (the scores come
    from the GPU's score kernel: top-k and expansion are exact functions of
    them, so the comparison is bit-exact)."""
    rows = list(rows)
    ref_ids = O.topk_pools(scores[rows], K)
    np.testing.assert_array_equal(ids[rows], ref_ids)
    ref_tok = O.expand_selection(ref_ids, np.asarray(row_seq)[rows], pool_start, kp, W)
    np.testing.assert_array_equal(tok[rows], ref_tok)


@pytest.mark.parametrize("Q,P,B", [(1000, 20000, 2), (4, 65536, 4), (9, 3000, 3), (835, 20000, 2), (100, 20000, 2),
                                   (8387, 2000, 2)])
def test_streamed_index_topk_bit_identical(Q, P, B):
    # dsa_index_topk_pools_expand gives the bits of dsa_index_scores +
    # dsa_topk_pools_expand, and those of the oracle's top-k and expansion of
    # the same scores: 1000 and 835 rows take the filtered path (5 pool ranges
    # per row, rows of two sequences in one workgroup; 835 leaves the last
    # workgroup partial); 4 (decode rows: one block with the split top-k), 9
    # and 100 rows (40 pool ranges per row would outgrow the scores) take the
    # row-blocked path, as do 8387 rows of 2000 pools (a 2048-key list would
    # outgrow the row): blocks of 8384 rows and a last block of 3 that takes
    # the decode score kernel
    rng = np.random.default_rng(Q + P)
    H, D, kp, K = 32, 128, 4, 512
    W = K * kp + 3
    k_pool = torch.from_numpy(rng.standard_normal((B, P, D)).astype(np.float32)).to(torch.bfloat16)
    q = torch.from_numpy(rng.standard_normal((Q, H, D)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.random((Q, H)) / H).astype(np.float32))
    gamma = torch.from_numpy((1 + 0.02 * rng.standard_normal(D)).astype(np.float32))
    beta = torch.from_numpy((0.02 * rng.standard_normal(D)).astype(np.float32))
    n = [P - 5 * b for b in range(B)]
    ps = np.full((B, P), -1, np.int32)
    pv = np.zeros((B, P), np.uint8)
    for b in range(B):
        ps[b, :n[b]] = 7 + kp * np.arange(n[b])
        pv[b, :n[b]] = rng.random(n[b]) > 0.02
    row_seq = np.sort(rng.integers(0, B, Q)).astype(np.int32)
    row_pos = (7 + kp * np.asarray(n)[row_seq] - rng.integers(0, 40, Q)).astype(np.int32)
    args = (dev(q), dev(w), D ** -0.5, dev(tile_pool_cache(k_pool)), dev(torch.from_numpy(ps)),
            dev(torch.from_numpy(pv)), dev(gamma), dev(beta), 1e-5, dev(torch.from_numpy(row_seq)),
            dev(torch.from_numpy(row_pos)), kp)
    scores = ops().dsa_index_scores(*args)
    ids_a, tok_a = ops().dsa_topk_pools_expand(scores, K, args[9], args[4], kp, W)
    ws = ops().topk_workspace(ops().dsa_index_topk_workspace_bytes(Q, P, K))
    for _ in range(2):   # twice on one workspace: the top-k counters are left zero
        ids_b, tok_b = ops().dsa_index_topk_pools_expand(*args, K, W, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(ids_a, ids_b)
        assert torch.equal(tok_a, tok_b)
    # against the oracle on the GPU's scores: the first rows, the last rows
    # (the ragged last block) and a sample
    rows = sorted(set([0, 1, Q // 2] + list(range(max(0, Q - 4), Q)) + rng.integers(0, Q, 4).tolist()))
    _streamed_vs_oracle(scores.cpu().numpy(), ids_b.cpu().numpy(), tok_b.cpu().numpy(), rows, row_seq, ps, kp, K, W)


def test_streamed_index_topk_prefill_chunk_full_size():
    # the prefill chunk (4096 rows x 32768 pools, forced ties at the cut): the
    # filtered path (one candidate list of 2048 keys per row), bit-identical to
    # the unfused calls and, on sampled rows (row 0, row 4095 and rows of
    # several workgroups), to the oracle's top-k and expansion of the GPU's
    # scores
    d = wl_data_prefill()
    wl, ip = d["wl"], d["ip"]
    pc = scores_inputs(d, k_pool_override=synth.codebook_keys(wl))
    args = (dev(ip["q"]), dev(ip["w"]), ip["scale"], dev(tile_pool_cache(pc["k_pool"])), dev(pc["pool_start"]),
            dev(pc["pool_valid"]), dev(ip["gamma"]), dev(ip["beta"]), ip["eps"], dev(ip["row_seq"]),
            dev(ip["row_pos"]), wl.kp)
    scores = ops().dsa_index_scores(*args)
    ids_a, tok_a = ops().dsa_topk_pools_expand(scores, wl.K, args[9], args[4], wl.kp, wl.W)
    rows = [0, 511, 512, 1023, 2047, 2048, 3000, 3583, 3584, 4095]
    s_rows = scores[rows].cpu().numpy()
    del scores
    ids_b, tok_b = ops().dsa_index_topk_pools_expand(*args, wl.K, wl.W)
    torch.cuda.synchronize()
    assert torch.equal(ids_a, ids_b)
    assert torch.equal(tok_a, tok_b)
    full = np.zeros((wl.Q, wl.P_max), np.float32)
    full[rows] = s_rows
    _streamed_vs_oracle(full, ids_b.cpu().numpy(), tok_b.cpu().numpy(), rows, ip["row_seq"].numpy(),
                        d["comp"]["pool_start"], wl.kp, wl.K, wl.W)


def _shaped_rows_inputs(kind: str, Q: int, P: int, B: int, H: int, seed: int):
    """Score-kernel inputs whose score rows take a chosen shape along the pool
    index: "rising" (every pool scores above the ones before it, up to small
    per-row wiggles: a candidate list keeps growing and is shrunk about every
    other stage), "falling", "equal" (all pools of a row score the same: the
    order is the pool index alone) and "codebook" (pooled keys drawn from 256
    rows: ~128-fold ties, as in the prefill chunk)."""
    rng = np.random.default_rng(seed)
    D, kp = 128, 4
    u = np.tile([1.0, -1.0], D // 2)            # zero-mean, orthogonal, |u|^2 = |v|^2 = D
    v = np.tile([1.0, 1.0, -1.0, -1.0], D // 4)
    if kind in ("rising", "falling"):
        t = np.arange(P) / (P - 1)
        theta = (np.pi / 2) * (1 - t if kind == "rising" else t)
        keys = np.cos(theta)[:, None] * u + np.sin(theta)[:, None] * v
    elif kind == "equal":
        keys = np.broadcast_to(u, (P, D))
    else:
        keys = rng.standard_normal((256, D))[rng.integers(0, 256, P)]
    k_pool = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(keys, (B, P, D)), np.float32)).to(torch.bfloat16)
    q = torch.from_numpy((u + 0.1 * rng.standard_normal((Q, H, D))).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((0.5 + rng.random((Q, H))).astype(np.float32) / H)
    gamma = torch.ones(D, dtype=torch.float32)
    beta = torch.zeros(D, dtype=torch.float32)
    ps = np.broadcast_to(7 + kp * np.arange(P, dtype=np.int32), (B, P)).copy()
    pv = (rng.random((B, P)) > 0.02).astype(np.uint8)
    row_seq = np.sort(rng.integers(0, B, Q)).astype(np.int32)
    # most rows see (nearly) every pool; a few see fewer than K candidates
    row_pos = (7 + kp * P - 1 - rng.integers(0, 400, Q)).astype(np.int32)
    row_pos[rng.integers(0, Q, 6)] = 7 + kp * rng.integers(0, 300, 6)
    args = (dev(q), dev(w), D ** -0.5, dev(tile_pool_cache(k_pool)), dev(torch.from_numpy(ps)),
            dev(torch.from_numpy(pv)), dev(gamma), dev(beta), 1e-5, dev(torch.from_numpy(row_seq)),
            dev(torch.from_numpy(row_pos)), kp)
    return args, row_seq, ps, kp


@pytest.mark.parametrize("kind,Q,P,H,K", [("rising", 4096, 32768, 32, 512), ("equal", 2048, 32768, 32, 512),
                                          ("falling", 1024, 32768, 16, 100), ("codebook", 2048, 32768, 32, 512),
                                          ("rising", 1024, 32768, 32, 1024), ("equal", 515, 20000, 16, 8),
                                          ("codebook", 600, 20003, 32, 512), ("rising", 2048, 32768, 32, 2048)])
def test_filtered_index_topk_shaped_score_rows(kind, Q, P, H, K):
    # the filtered path of dsa_index_topk_pools_expand (bf16, D = 128, H = 16
    # or 32, Q > 64: each score-kernel wave keeps a list of its row's
    # candidates over its pool range and shrinks it as it fills) gives the bits
    # of dsa_index_scores + dsa_topk_pools_expand and the oracle's top-k and
    # expansion of the same scores.  The cases cover 1 (4096 rows), 2, 4, 7
    # (600 rows of 20003 pools: a partial last tile) and 8 pool ranges per row
    # (515 rows, the last workgroup partial), K = 8 .. 2048 (lists of 8192 keys,
    # read over several rounds by a shrink)
    # (lists of 2048 and 4096 keys), and score rows that force shrinks every
    # other stage (rising), ties through the index bits (equal, codebook)
    args, row_seq, ps, kp = _shaped_rows_inputs(kind, Q, P, 2, H, seed=Q + K)
    W = K * kp + 5
    scores = ops().dsa_index_scores(*args)
    ids_a, tok_a = ops().dsa_topk_pools_expand(scores, K, args[9], args[4], kp, W)
    ws = ops().topk_workspace(ops().dsa_index_topk_workspace_bytes(Q, P, K))
    for _ in range(2):   # twice on one workspace: nothing of the first call's lists is read
        ids_b, tok_b = ops().dsa_index_topk_pools_expand(*args, K, W, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(ids_a, ids_b)
        assert torch.equal(tok_a, tok_b)
    rng = np.random.default_rng(Q)
    rows = sorted(set([0, Q - 1] + rng.integers(0, Q, 6).tolist()))
    s_np = scores[rows].cpu().numpy()
    full = np.zeros((Q, P), np.float32)
    full[rows] = s_np
    _streamed_vs_oracle(full, ids_b.cpu().numpy(), tok_b.cpu().numpy(), rows, row_seq, ps, kp, K, W)
    # the rows have the intended shape
    fin = [r[np.isfinite(r)] for r in s_np]
    if kind == "equal":
        assert all(len(f) and np.all(f == f[0]) for f in fin)
        ids = ids_b.cpu().numpy()
        for i, r in enumerate(rows):   # then the first K candidates by pool index
            cand = np.flatnonzero(np.isfinite(s_np[i]))[:K]
            np.testing.assert_array_equal(ids[r][:len(cand)], cand)
    elif kind in ("rising", "falling"):
        # rank correlation with the pool index (bf16 keys make the rows
        # staircases with small steps back, so not every step is up)
        for f in fin:
            if len(f) > 1000:
                rho = np.corrcoef(np.argsort(np.argsort(f, kind="stable")), np.arange(len(f)))[0, 1]
                assert rho > 0.95 if kind == "rising" else rho < -0.95


def test_streamed_index_topk_paths_share_one_workspace():
    # one workspace for both paths of dsa_index_topk_pools_expand, called in
    # turn: the filtered path (1000 rows of 20000 pools) writes its lists past
    # the top-k counter block and leaves that block zero, so the row-blocked
    # path's split top-k (4 decode rows of 65536 pools, whose merge counters
    # live there) still gives the unfused calls' bits, and so does the
    # filtered path after it
    cases = []
    for Q, P, B in ((1000, 20000, 2), (4, 65536, 4)):
        rng = np.random.default_rng(Q + 7)
        H, D, kp, K = 32, 128, 4, 512
        W = K * kp
        k_pool = torch.from_numpy(rng.standard_normal((B, P, D)).astype(np.float32)).to(torch.bfloat16)
        q = torch.from_numpy(rng.standard_normal((Q, H, D)).astype(np.float32)).to(torch.bfloat16)
        w = torch.from_numpy((rng.random((Q, H)) / H).astype(np.float32))
        gamma = torch.from_numpy((1 + 0.02 * rng.standard_normal(D)).astype(np.float32))
        beta = torch.from_numpy((0.02 * rng.standard_normal(D)).astype(np.float32))
        ps = np.broadcast_to(7 + kp * np.arange(P, dtype=np.int32), (B, P)).copy()
        pv = (rng.random((B, P)) > 0.02).astype(np.uint8)
        row_seq = np.sort(rng.integers(0, B, Q)).astype(np.int32)
        row_pos = (7 + kp * P - 1 - rng.integers(0, 40, Q)).astype(np.int32)
        args = (dev(q), dev(w), D ** -0.5, dev(tile_pool_cache(k_pool)), dev(torch.from_numpy(ps)),
                dev(torch.from_numpy(pv)), dev(gamma), dev(beta), 1e-5, dev(torch.from_numpy(row_seq)),
                dev(torch.from_numpy(row_pos)), kp)
        scores = ops().dsa_index_scores(*args)
        ref = ops().dsa_topk_pools_expand(scores, K, args[9], args[4], kp, W)
        cases.append((args, K, W, ref, ops().dsa_index_topk_workspace_bytes(Q, P, K)))
    ws = ops().topk_workspace(max(c[4] for c in cases))
    for args, K, W, (ids_a, tok_a), _ in cases + cases:
        ids_b, tok_b = ops().dsa_index_topk_pools_expand(*args, K, W, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(ids_a, ids_b)
        assert torch.equal(tok_a, tok_b)
    from dsa_decode_amd._lib import DSA_TOPK_COUNTER_BYTES
    assert not ws[:DSA_TOPK_COUNTER_BYTES].any()


def test_bound_call_keeps_its_buffers_and_sizes_its_workspace():
    # a pre-bound top-k made from temporaries (output created inline, no
    # workspace given, on the decode shape whose split rows need a workspace)
    # holds those buffers for as long as the call exists, so new allocations
    # cannot land on them, and writes what the entry point writes
    import gc
    import weakref
    s = dev(synth.random_scores(4, 65536, seed=12, tie_levels=20))
    ref = ops().dsa_topk_pools(s, 512)
    out = torch.full((4, 512), 0x7fffffff, dtype=torch.int32, device="cuda")
    call = ops().bind_topk_pools(s, 512, out.clone(), None)
    held = [weakref.ref(t) for t in call.keep]
    assert len(held) == 3                       # scores, pool_ids, the workspace made for the call
    gc.collect()
    junk = [torch.full((1 << 18,), -7, dtype=torch.int32, device="cuda") for _ in range(32)]
    for _ in range(2):
        call()
        torch.cuda.synchronize()
        assert torch.equal(call.keep[1], ref)
    assert all(h() is not None for h in held)
    del call, junk
    gc.collect()
    assert held[2]() is None                    # the call's own workspace goes with it
