"""GPU parity of the per-sequence indexer state (dsa_kpool_append) and of a
whole decode step captured in a HIP graph.

The state's definition is the compress of the sequence at its current length
(page "Module glm5next_dsa": module "state", and the compress rules of
"Traps carried from Slice 8"), so the oracle here is the oracle's
kpool_compress at that length.  Bars: integer state exact; pooled keys bit-equal
to the GPU's full compress (same per-pool arithmetic) and within the compress
tolerance of the oracle; graph replays bit-equal to the same calls run eagerly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from dsa_decode_amd import synth
from oracle import dsa_oracle as O
from tests.helpers import assert_compress_close, dev, untile_pool_cache

pytestmark = pytest.mark.gpu


def ops():
    from dsa_decode_amd import ops as _ops
    return _ops


def _inputs(B, T, D, kp, dtype, seed):
    rng = np.random.default_rng(seed)
    k = torch.from_numpy(rng.standard_normal((B, T, D)).astype(np.float32)).to(dtype)
    gate = torch.from_numpy(rng.standard_normal((B, T, D)).astype(np.float32)).to(dtype)
    ape = torch.from_numpy((0.1 * rng.standard_normal((kp, D))).astype(np.float32))
    valid = np.ones((B, T), np.uint8)
    valid[0, :5] = 0                      # left padding
    if B > 1:
        valid[1, :37] = 0                 # padding longer than several pools
        valid[1, 50] = 0                  # a hole
    if B > 2:
        valid[2, :] = 0                   # nothing valid for a while, then valid
        valid[2, 61:] = 1
    return k, gate, torch.from_numpy(valid), ape


def _state_equal(a: dict, b: dict) -> None:
    for name in ("n_pools", "first_valid", "pool_start", "pool_valid"):
        np.testing.assert_array_equal(a[name].cpu().numpy(), b[name].cpu().numpy(), err_msg=name)
    ga, gb = a["k_pool"].cpu(), b["k_pool"].cpu()
    assert torch.equal(ga.view(torch.int16) if ga.dtype == torch.bfloat16 else ga.view(torch.int32),
                       gb.view(torch.int16) if gb.dtype == torch.bfloat16 else gb.view(torch.int32))


def _empty_state(k, gate, valid, ape, kp, P_max):
    B = k.shape[0]
    return ops().dsa_kpool_compress(dev(k), dev(gate), dev(valid), dev(ape),
                                    dev(torch.zeros(B, dtype=torch.int32)), kp, P_max)


@pytest.mark.parametrize("kp,D,dtype", [(4, 128, torch.bfloat16), (1, 32, torch.float32),
                                        (3, 64, torch.bfloat16), (8, 128, torch.bfloat16)])
def test_append_in_steps_matches_full_compress_and_oracle(kp, D, dtype):
    B, T = 3, 160
    P_max = T // kp + 1
    k, gate, valid, ape = _inputs(B, T, D, kp, dtype, seed=kp)
    kd, gd, vd, ad = dev(k), dev(gate), dev(valid), dev(ape)
    state = _empty_state(k, gate, valid, ape, kp, P_max)
    rng = np.random.default_rng(100 + kp)
    L = np.zeros(B, np.int32)
    checks = 0
    while (L < T).any():
        # each sequence grows by 0..3 tokens (mostly one), independently
        L = np.minimum(T, L + rng.choice([0, 1, 1, 1, 2, 3], size=B)).astype(np.int32)
        ops().dsa_kpool_append(kd, gd, vd, ad, dev(torch.from_numpy(L)), kp, state, max_new_pools=1)
        if rng.random() < 0.15 or (L == T).all():
            # drain any backlog (max_new_pools = 1 forms at most one pool per call,
            # so the state may lag); each call continues where the last stopped
            for _ in range(P_max):
                before = state["n_pools"].clone()
                ops().dsa_kpool_append(kd, gd, vd, ad, dev(torch.from_numpy(L)), kp, state, max_new_pools=2)
                if torch.equal(before, state["n_pools"]):
                    break
            full = ops().dsa_kpool_compress(kd, gd, vd, ad, dev(torch.from_numpy(L)), kp, P_max)
            torch.cuda.synchronize()
            _state_equal(state, full)
            checks += 1
    assert checks >= 2
    # the final state against the oracle's compress of the whole sequences
    ref = O.kpool_compress(k, gate, valid, ape, torch.from_numpy(L), kp, P_max)
    np.testing.assert_array_equal(state["n_pools"].cpu().numpy(), ref["n_pools"])
    np.testing.assert_array_equal(state["first_valid"].cpu().numpy(), ref["first_valid"])
    np.testing.assert_array_equal(state["pool_start"].cpu().numpy(), ref["pool_start"])
    np.testing.assert_array_equal(state["pool_valid"].cpu().numpy().astype(bool), ref["pool_valid"])
    absk = O.kpool_compress(k.abs(), gate, valid, ape, torch.from_numpy(L), kp, P_max)["k_pool"]
    assert_compress_close(untile_pool_cache(state["k_pool"].cpu(), P_max), ref["k_pool"], absk, dtype)


def test_append_backlog_bound_and_large_jumps():
    # one call that appends many tokens forms at most max_new_pools pools; the
    # next calls continue where it stopped; with a large bound one call suffices
    kp, D, dtype, B, T = 4, 128, torch.bfloat16, 3, 300
    P_max = T // kp
    k, gate, valid, ape = _inputs(B, T, D, kp, dtype, seed=7)
    kd, gd, vd, ad = dev(k), dev(gate), dev(valid), dev(ape)
    Ld = dev(torch.full((B,), T, dtype=torch.int32))
    full = ops().dsa_kpool_compress(kd, gd, vd, ad, Ld, kp, P_max)
    st = _empty_state(k, gate, valid, ape, kp, P_max)
    ops().dsa_kpool_append(kd, gd, vd, ad, Ld, kp, st, max_new_pools=10)
    n1 = st["n_pools"].cpu().numpy()
    assert (n1 <= 10).all() and (n1 == np.minimum(10, full["n_pools"].cpu().numpy())).all()
    for _ in range(8):
        ops().dsa_kpool_append(kd, gd, vd, ad, Ld, kp, st, max_new_pools=10)
    torch.cuda.synchronize()
    _state_equal(st, full)
    st2 = _empty_state(k, gate, valid, ape, kp, P_max)
    ops().dsa_kpool_append(kd, gd, vd, ad, Ld, kp, st2, max_new_pools=P_max)
    torch.cuda.synchronize()
    _state_equal(st2, full)


def test_append_shrunk_length_clears_rows():
    # a length that shrank (a precondition violation) leaves the state of a
    # full compress at the shorter length, never stale pools
    kp, D, dtype, B, T = 4, 32, torch.float32, 3, 120
    P_max = T // kp
    k, gate, valid, ape = _inputs(B, T, D, kp, dtype, seed=9)
    kd, gd, vd, ad = dev(k), dev(gate), dev(valid), dev(ape)
    st = ops().dsa_kpool_compress(kd, gd, vd, ad, dev(torch.full((B,), T, dtype=torch.int32)), kp, P_max)
    L = dev(torch.tensor([90, 100, 110], dtype=torch.int32))
    ops().dsa_kpool_append(kd, gd, vd, ad, L, kp, st, max_new_pools=1)
    full = ops().dsa_kpool_compress(kd, gd, vd, ad, L, kp, P_max)
    torch.cuda.synchronize()
    _state_equal(st, full)


def test_decode_step_in_a_hip_graph_matches_eager():
    """One decode step (append the new token -> scores -> top-k + expand ->
    sparse MLA) captured once in a HIP graph and replayed for 9 consecutive
    tokens (crossing pool boundaries), with the host writing the new length
    and position between replays.  Every replay's outputs and the advanced
    state are bit-equal to the same calls run eagerly on a twin state, and the
    final state equals a full compress at the final length."""
    wl = synth.workload("decode")
    ti = synth.token_inputs(wl)
    ip = synth.index_params(wl)
    mi = synth.mla_inputs(wl)
    kp, K, W, T = wl.kp, wl.K, wl.W, wl.T_max
    L0 = T - 10
    kd, gd, vd, ad = dev(ti["k"]), dev(ti["gate"]), dev(ti["valid"]), dev(ti["ape"])
    q, w, ga, be = dev(ip["q"]), dev(ip["w"]), dev(ip["gamma"]), dev(ip["beta"])
    rs = dev(ip["row_seq"])
    ql, kv = dev(mi["q_lat"]), dev(mi["kv"])
    P_max, Q = wl.P_max, wl.Q

    def make_side():
        L = dev(torch.full((wl.B,), L0, dtype=torch.int32))
        st = ops().dsa_kpool_compress(kd, gd, vd, ad, L, kp, P_max)
        lib = ops()._lib.load()
        side = dict(
            L=L, pos=dev(torch.full((Q,), L0 - 1, dtype=torch.int32)), st=st,
            scores=torch.empty((Q, P_max), dtype=torch.float32, device="cuda"),
            ids=torch.empty((Q, K), dtype=torch.int32, device="cuda"),
            tok=torch.empty((Q, W), dtype=torch.int32, device="cuda"),
            out=torch.empty((Q, wl.Hm, wl.Dl), dtype=torch.bfloat16, device="cuda"),
            lse=torch.empty((Q, wl.Hm), dtype=torch.float32, device="cuda"),
            tws=ops().topk_workspace(lib.dsa_topk_workspace_bytes(Q, P_max, K)),
            mws=torch.zeros(max(1, lib.dsa_sparse_mla_workspace_bytes(Q, wl.Hm, wl.Dl, W, 1)),
                            dtype=torch.uint8, device="cuda"))
        return side

    def step(s):
        ops().dsa_kpool_append(kd, gd, vd, ad, s["L"], kp, s["st"], max_new_pools=1)
        ops().dsa_index_scores(q, w, ip["scale"], s["st"]["k_pool"], s["st"]["pool_start"], s["st"]["pool_valid"],
                               ga, be, ip["eps"], rs, s["pos"], kp, scores=s["scores"])
        ops().dsa_topk_pools_expand(s["scores"], K, rs, s["st"]["pool_start"], kp, W, pool_ids=s["ids"],
                                    token_ids=s["tok"], workspace=s["tws"])
        ops().dsa_sparse_mla_decode(ql, kv, rs, s["tok"], mi["sm_scale"], out=s["out"], lse=s["lse"],
                                    workspace=s["mws"])

    g_side, e_side = make_side(), make_side()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step(g_side)           # warm-up outside capture (the length is still L0: no new pool)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step(g_side)
    torch.cuda.synchronize()
    for i in range(1, 10):
        L = L0 + i
        for s in (g_side, e_side):
            s["L"].fill_(L)
            s["pos"].fill_(L - 1)
        torch.cuda.synchronize()
        graph.replay()
        step(e_side)
        torch.cuda.synchronize()
        _state_equal(g_side["st"], e_side["st"])
        for name in ("scores", "ids", "tok", "lse"):
            assert torch.equal(g_side[name], e_side[name]), (i, name)
        assert torch.equal(g_side["out"].view(torch.int16), e_side["out"].view(torch.int16)), i
        # the newest whole pool is a candidate exactly when its last token is the current one or earlier
        n = int(g_side["st"]["n_pools"][0])
        assert n == L // kp
        assert np.isfinite(g_side["scores"][0, n - 1].item())
    full = ops().dsa_kpool_compress(kd, gd, vd, ad, g_side["L"], kp, P_max)
    torch.cuda.synchronize()
    _state_equal(g_side["st"], full)
