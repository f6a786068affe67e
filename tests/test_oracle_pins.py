"""Pins of the CPU oracle against facts that do not come from the oracle itself:
values the pages state, closed forms, special cases that reduce to a library
routine (torch / scipy), brute force on tiny inputs and invariants.  CPU only.
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

from oracle import dsa_oracle as O
from dsa_decode_amd import synth
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _mk_tokens(T, pad, kp, D, seed, B=1, holes=()):
    r = _rng(seed)
    k = r.standard_normal((B, T, D))
    gate = r.standard_normal((B, T, D))
    ape = 0.1 * r.standard_normal((kp, D))
    valid = np.zeros((B, T), np.uint8)
    valid[:, pad:T] = 1
    for (b, t) in holes:
        valid[b, t] = 0
    return k, gate, valid, ape, np.full(B, T)


# ---------------------------------------------------------------- compress
def _golden_pool_counts():
    rows = []
    for line in open(os.path.join(GOLDEN, "pool_counts.txt")):
        if line.startswith("#") or not line.strip():
            continue
        f = line.split()
        rows.append(tuple(int(x) for x in f[:5]))
    return rows


@pytest.mark.parametrize("T,pad,kp,n_exp,first_exp", _golden_pool_counts())
def test_pool_count_golden(T, pad, kp, n_exp, first_exp):
    valid = np.zeros(T, np.uint8)
    valid[pad:] = 1
    f, n = O.anchor(valid, T, kp)
    assert (n, f) == (n_exp, first_exp)


def test_tiny_workload_pools_anchor_and_tail():
    wl = synth.workload("tiny")
    ti = synth.token_inputs(wl)
    out = O.kpool_compress(ti["k"], ti["gate"], ti["valid"], ti["ape"], ti["seq_len"], wl.kp, wl.P_max)
    assert out["n_pools"].tolist() == [62] and out["first_valid"].tolist() == [5]
    assert out["pool_start"][0, :62].tolist() == [5 + 4 * p for p in range(62)]
    assert out["pool_valid"][0, :62].all()
    # the trailing partial pool (tokens 253..255) and the unused row are not pools
    assert (out["pool_start"][0, 62:] == -1).all() and not out["pool_valid"][0, 62:].any()
    assert (out["k_pool"][0, 62:] == 0).all()


def test_kpool_one_is_identity():
    k, gate, valid, ape, L = _mk_tokens(40, 3, 1, 8, 1)
    out = O.kpool_compress(k, gate, valid, ape, L, 1, 40)
    assert out["n_pools"][0] == 37
    np.testing.assert_array_equal(out["k_pool"][0, :37], k[0, 3:40])


def test_equal_logits_give_slot_mean():
    kp, D, pad, T = 4, 8, 5, 45
    k, gate, valid, ape, L = _mk_tokens(T, pad, kp, D, 2)
    c = _rng(3).standard_normal(D)
    for t in range(pad, T):
        s = (t - pad) % kp
        gate[0, t] = c - ape[s]              # every slot logit equals c
    out = O.kpool_compress(k, gate, valid, ape, L, kp, T // kp)
    n = (T - pad) // kp
    mean = k[0, pad:pad + n * kp].reshape(n, kp, D).mean(axis=1)
    np.testing.assert_allclose(out["k_pool"][0, :n], mean, rtol=1e-13, atol=1e-14)


def test_dominant_logit_selects_its_slot():
    kp, D, pad, T = 4, 8, 2, 34
    k, gate, valid, ape, L = _mk_tokens(T, pad, kp, D, 4)
    for t in range(pad, T):
        if (t - pad) % kp == 2:
            gate[0, t] += 60.0
    out = O.kpool_compress(k, gate, valid, ape, L, kp, T // kp)
    n = (T - pad) // kp
    np.testing.assert_allclose(out["k_pool"][0, :n], k[0, pad + 2:pad + n * kp:kp], atol=1e-20, rtol=1e-20 + 1e-24)


def test_softmax_weights_match_scipy_over_slot_axis():
    # one-hot keys: token in slot s carries 1 in channels c with c % kp == s, so
    # k_pool[p, c] is the weight of slot c % kp in channel c.  Anchor not on a
    # multiple of kp, so a slot index taken from the absolute token would fail.
    kp, D, pad, T = 4, 12, 3, 43
    _, gate, valid, ape, L = _mk_tokens(T, pad, kp, D, 5)
    k = np.zeros_like(gate)
    for t in range(pad, T):
        s = (t - pad) % kp
        k[0, t, [c for c in range(D) if c % kp == s]] = 1.0
    out = O.kpool_compress(k, gate, valid, ape, L, kp, T // kp)
    n = (T - pad) // kp
    logits = gate[0, pad:pad + n * kp].reshape(n, kp, D) + ape[None]
    wts = scipy.special.softmax(logits, axis=1)          # [n, kp, D]
    expect = np.stack([wts[:, c % kp, c] for c in range(D)], axis=1)
    np.testing.assert_allclose(out["k_pool"][0, :n], expect, rtol=1e-13)


def test_holes_invalidate_only_their_pool():
    kp, D, pad, T = 4, 4, 5, 45
    k, gate, valid, ape, L = _mk_tokens(T, pad, kp, D, 6, holes=[(0, 5 + 4 * 3 + 2)])
    out = O.kpool_compress(k, gate, valid, ape, L, kp, T // kp)
    assert out["first_valid"][0] == 5 and out["n_pools"][0] == 10
    assert out["pool_valid"][0, :10].tolist() == [True] * 3 + [False] + [True] * 6


def test_hole_at_anchor_moves_anchor():
    kp, D, T = 4, 4, 40
    k, gate, valid, ape, L = _mk_tokens(T, 0, kp, D, 7, holes=[(0, 0), (0, 1)])
    out = O.kpool_compress(k, gate, valid, ape, L, kp, T // kp)
    assert out["first_valid"][0] == 2 and out["n_pools"][0] == 9
    assert out["pool_start"][0, :9].tolist() == [2 + 4 * p for p in range(9)]


def test_all_invalid_sequence_has_no_pools():
    k, gate, valid, ape, L = _mk_tokens(32, 32, 4, 4, 8)
    out = O.kpool_compress(k, gate, valid, ape, L, 4, 8)
    assert out["n_pools"][0] == 0
    assert (out["pool_start"] == -1).all() and not out["pool_valid"].any() and (out["k_pool"] == 0).all()


def test_kpool_limit_from_pages():
    lim = dict(l.split() for l in open(os.path.join(GOLDEN, "limits.txt")) if l.strip() and not l.startswith("#"))
    assert O.MAX_KPOOL == int(lim["max_kpool"])
    k, gate, valid, ape, L = _mk_tokens(64, 0, 9, 4, 9)
    with pytest.raises(ValueError):
        O.kpool_compress(k, gate, valid, ape, L, 9, 64)
    k, gate, valid, ape, L = _mk_tokens(64, 0, 8, 4, 9)
    assert O.kpool_compress(k, gate, valid, ape, L, 8, 8)["n_pools"][0] == 8


# ---------------------------------------------------------------- layer norm + scores
def test_layer_norm_matches_torch():
    r = _rng(10)
    x = r.standard_normal((17, 24)) * 3 + 0.7
    g = 1 + 0.02 * r.standard_normal(24)
    b = 0.02 * r.standard_normal(24)
    ref = F.layer_norm(torch.from_numpy(x), (24,), torch.from_numpy(g), torch.from_numpy(b), 1e-5).numpy()
    np.testing.assert_allclose(O.layer_norm(x, g, b, 1e-5), ref, rtol=1e-12, atol=1e-12)


def _score_setup(P=40, D=16, H=1, Q=1, B=1, seed=11):
    r = _rng(seed)
    k_pool = r.standard_normal((B, P, D))
    gamma = 1 + 0.02 * r.standard_normal(D)
    beta = 0.02 * r.standard_normal(D)
    q = r.standard_normal((Q, H, D))
    pool_start = np.tile(np.arange(P) * 4, (B, 1))
    pool_valid = np.ones((B, P), bool)
    return k_pool, gamma, beta, q, pool_start, pool_valid


def _torch_dots(k_pool_b, gamma, beta, q_rows):
    kn = F.layer_norm(torch.from_numpy(k_pool_b), (k_pool_b.shape[-1],), torch.from_numpy(gamma),
                      torch.from_numpy(beta), 1e-5)
    return torch.einsum("pd,hd->ph", kn, torch.from_numpy(q_rows)).numpy()


def test_single_head_score_is_scaled_normed_dot():
    k_pool, gamma, beta, q, ps, pv = _score_setup()
    scale = 0.25
    s = O.index_scores(q, np.ones((1, 1)), scale, k_pool, ps, pv, gamma, beta, 1e-5,
                       [0], [10 ** 6], 4)[0]
    dots = _torch_dots(k_pool[0], gamma, beta, q[0])[:, 0]
    expect = np.where(dots > 0, scale * dots, 0.0)
    np.testing.assert_allclose(s, expect, rtol=1e-6, atol=1e-7)
    assert (dots > 0).any() and (dots < 0).any()


def test_relu_pair_gives_absolute_value():
    k_pool, gamma, beta, q, ps, pv = _score_setup(H=1, seed=12)
    q2 = np.concatenate([q, -q], axis=1)               # heads h and -h
    s = O.index_scores(q2, np.ones((1, 2)), 0.5, k_pool, ps, pv, gamma, beta, 1e-5, [0], [10 ** 6], 4)[0]
    dots = _torch_dots(k_pool[0], gamma, beta, q[0])[:, 0]
    np.testing.assert_allclose(s, 0.5 * np.abs(dots), rtol=1e-6, atol=1e-7)


def test_head_weights_are_per_row_and_head():
    Q, H = 3, 5
    k_pool, gamma, beta, q, ps, pv = _score_setup(H=H, Q=Q, seed=13)
    dots = [_torch_dots(k_pool[0], gamma, beta, q[r]) for r in range(Q)]
    for r in range(Q):
        for h in range(H):
            w = np.zeros((Q, H))
            w[r, h] = 0.7
            s = O.index_scores(q, w, 0.3, k_pool, ps, pv, gamma, beta, 1e-5, [0] * Q, [10 ** 6] * Q, 4)
            np.testing.assert_allclose(s[r], 0.7 * np.maximum(0, 0.3 * dots[r][:, h]), rtol=1e-6, atol=1e-7)
            others = [x for x in range(Q) if x != r]
            assert (s[others] == 0).all()


def test_scores_scale_linearly_in_w():
    k_pool, gamma, beta, q, ps, pv = _score_setup(H=4, Q=2, seed=14)
    w = _rng(15).random((2, 4))
    a = O.index_scores(q, w, 0.2, k_pool, ps, pv, gamma, beta, 1e-5, [0, 0], [10 ** 6] * 2, 4)
    b = O.index_scores(q, 4.0 * w, 0.2, k_pool, ps, pv, gamma, beta, 1e-5, [0, 0], [10 ** 6] * 2, 4)
    np.testing.assert_array_equal(b, 4.0 * a)       # power-of-two scaling is exact


def test_candidate_rule_causal_boundary_and_validity():
    P, kp = 12, 4
    k_pool, gamma, beta, q, ps, pv = _score_setup(P=P, H=2, Q=3, seed=16)
    pv[0, 3] = False
    ps[0, 10:] = -1
    pv[0, 10:] = False
    pos = [ps[0, 6] + kp - 1, ps[0, 6] + kp - 2, 10 ** 6]
    s = O.index_scores(q, np.ones((3, 2)), 0.5, k_pool, ps, pv, gamma, beta, 1e-5, [0] * 3, pos, kp)
    fin = np.isfinite(s)
    assert fin[0].tolist() == [p <= 6 and p != 3 for p in range(P)]
    assert fin[1].tolist() == [p <= 5 and p != 3 for p in range(P)]
    assert fin[2].tolist() == [p < 10 and p != 3 for p in range(P)]
    assert (s[~fin] == -np.inf).all()


def test_rows_read_their_own_sequence():
    k_pool, gamma, beta, q, ps, pv = _score_setup(H=3, Q=2, B=2, seed=17)
    w = np.ones((2, 3))
    both = O.index_scores(q, w, 0.5, k_pool, ps, pv, gamma, beta, 1e-5, [1, 0], [10 ** 6] * 2, 4)
    one = O.index_scores(q[:1], w[:1], 0.5, k_pool[1:], ps[1:], pv[1:], gamma, beta, 1e-5, [0], [10 ** 6], 4)
    np.testing.assert_array_equal(both[0], one[0])


# ---------------------------------------------------------------- top-k
def _brute_topk(s, K):
    """Rank by counting: rank(p) = #{p' beating p}; O(P^2), tiny rows only."""
    P = len(s)
    cand = [p for p in range(P) if s[p] != -np.inf]
    out = [-1] * K
    for p in cand:
        rank = sum(1 for p2 in cand if (s[p2] > s[p]) or (s[p2] == s[p] and p2 < p))
        if rank < K:
            out[rank] = p
    return out


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_rank_counting(seed):
    s = synth.random_scores(4, 97, seed, tie_levels=7, neg_inf_frac=0.2, signed_zeros=True).numpy()
    s[1, :] = -np.inf
    s[2, 5:] = -np.inf                                # fewer candidates than K
    K = 9
    got = O.topk_pools(s, K)
    for r in range(4):
        assert got[r].tolist() == _brute_topk(s[r], K)


def test_topk_tie_free_equals_torch_topk():
    s = synth.random_scores(3, 500, 3).numpy()
    got = O.topk_pools(s, 32)
    ref = torch.topk(torch.from_numpy(s), 32, dim=1, sorted=True).indices.numpy()
    np.testing.assert_array_equal(got, ref)


def test_topk_signed_zero_tie_and_padding():
    s = np.array([[-0.0, 0.0, -1.0, -np.inf, -0.0]], np.float32)
    assert O.topk_pools(s, 6).tolist() == [[0, 1, 4, 2, -1, -1]]


# ---------------------------------------------------------------- expand
def test_expand_worked_example():
    kv = {}
    for line in open(os.path.join(GOLDEN, "expand_example.txt")):
        if line.startswith("#") or not line.strip():
            continue
        f = line.split()
        kv[f[0]] = [int(x) for x in f[1:]]
    kp, W = kv["kpool"][0], kv["out_width"][0]
    tok = O.expand_selection(np.array([kv["pool_ids"]]), [0], np.array([kv["pool_start"]]), kp, W)
    assert tok[0].tolist() == kv["token_ids"]


def test_expand_invariants_on_tiny_workload():
    wl = synth.workload("tiny")
    ti = synth.token_inputs(wl)
    comp = O.kpool_compress(ti["k"], ti["gate"], ti["valid"], ti["ape"], ti["seq_len"], wl.kp, wl.P_max)
    s = synth.random_scores(1, wl.P_max, 5).numpy()
    s[:, comp["n_pools"][0]:] = -np.inf
    ids = O.topk_pools(s, wl.K)
    W = wl.W + 5
    tok = O.expand_selection(ids, [0], comp["pool_start"], wl.kp, W)[0]
    live = tok[tok >= 0]
    assert live.size == wl.K * wl.kp and (tok[wl.K * wl.kp:] == -1).all()
    assert len(set(live.tolist())) == live.size
    assert ((live >= 5) & (live < 5 + 62 * 4)).all()
    assert set(((live - 5) // 4).tolist()) == set(ids[0].tolist())
    with pytest.raises(ValueError):
        O.expand_selection(ids, [0], comp["pool_start"], wl.kp, wl.W - 1)


# ---------------------------------------------------------------- sparse MLA
def _mla_setup(T=50, Hm=3, Dl=16, seed=20):
    r = _rng(seed)
    return r.standard_normal((1, Hm, Dl)), r.standard_normal((1, T, Dl))


def _sdpa(q, kv, scale, mask=None):
    qt = torch.from_numpy(q)[:, :, None, :].transpose(1, 2)   # [1, 1, Hm, Dl] -> heads as batch below
    qh = torch.from_numpy(q[0])[:, None, :]                  # [Hm, 1, Dl]
    k = torch.from_numpy(kv[0])[None].expand(q.shape[1], -1, -1)   # [Hm, T, Dl]
    m = None if mask is None else torch.from_numpy(mask)[None, None, :].expand(q.shape[1], 1, -1)
    o = F.scaled_dot_product_attention(qh, k, k, attn_mask=m, scale=scale)
    del qt
    return o[:, 0, :].numpy()


def test_mla_full_selection_is_dense_attention():
    q, kv = _mla_setup()
    ids = np.arange(50)[None]
    out, lse = O.sparse_mla_decode(q, kv, [0], ids, 0.25)
    np.testing.assert_allclose(out[0], _sdpa(q, kv, 0.25), rtol=1e-10, atol=1e-12)
    logits = 0.25 * torch.from_numpy(q[0]) @ torch.from_numpy(kv[0]).T
    np.testing.assert_allclose(lse[0], torch.logsumexp(logits, dim=1).numpy(), rtol=1e-12)


def test_mla_selection_is_masked_dense_attention():
    q, kv = _mla_setup(seed=21)
    sel = np.array([3, 17, 4, -1, 40, 22, -1, 9])
    out, _ = O.sparse_mla_decode(q, kv, [0], sel[None], 0.3)
    mask = np.zeros(50, bool)
    mask[sel[sel >= 0]] = True
    np.testing.assert_allclose(out[0], _sdpa(q, kv, 0.3, mask), rtol=1e-10, atol=1e-12)


def test_mla_permutation_single_empty_and_hull():
    q, kv = _mla_setup(seed=22)
    sel = np.array([5, 6, 30, 2, 11])
    a, la = O.sparse_mla_decode(q, kv, [0], sel[None], 0.2)
    b, lb = O.sparse_mla_decode(q, kv, [0], sel[::-1].copy()[None], 0.2)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(la, lb, rtol=1e-14)
    lo, hi = kv[0, sel].min(axis=0), kv[0, sel].max(axis=0)
    assert ((a[0] >= lo - 1e-12) & (a[0] <= hi + 1e-12)).all()
    one, l1 = O.sparse_mla_decode(q, kv, [0], np.array([[-1, 7, -1]]), 0.2)
    np.testing.assert_allclose(one[0], np.tile(kv[0, 7], (3, 1)), rtol=1e-14)
    np.testing.assert_allclose(l1[0], 0.2 * q[0] @ kv[0, 7], rtol=1e-13)
    z, lz = O.sparse_mla_decode(q, kv, [0], np.array([[-1, -1]]), 0.2)
    assert (z == 0).all() and (lz == -np.inf).all()


# ---------------------------------------------------------------- rounding helpers
def test_round_bf16_matches_torch_on_fp32_values_and_ties():
    r = _rng(30)
    x = r.standard_normal(10000).astype(np.float32) * np.float32(3.0)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(O.round_bf16(x.astype(np.float64)), ref)
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130 + 2 ** -134])
    np.testing.assert_array_equal(O.round_bf16(ties), np.array([1.0, 1 + 2 ** -6, -1.0, 2 ** -130], np.float32))


# ---------------------------------------------------------------- workload properties
def test_prefill_workload_has_ties_straddling_the_cut():
    wl = synth.workload("prefill")
    ip = synth.index_params(wl)
    kpool = synth.codebook_keys(wl)
    P = wl.P_max
    ps = np.arange(P)[None] * wl.kp
    pv = np.ones((1, P), bool)
    rows = [0, 2047, 4095]
    s = O.index_scores(ip["q"], ip["w"], ip["scale"], kpool, ps, pv, ip["gamma"], ip["beta"], ip["eps"],
                       ip["row_seq"], ip["row_pos"], wl.kp, rows=rows)
    straddle = 0
    for i in range(len(rows)):
        v = np.sort(s[i][np.isfinite(s[i])])[::-1]
        straddle += int(v[wl.K - 1] == v[wl.K])
        assert 31744 <= np.isfinite(s[i]).sum() <= 32768
    assert straddle >= 2


def test_expand_rows_use_their_own_sequence():
    pool_start = np.array([[0, 4, 8, 12], [3, 7, 11, 15]])
    tok = O.expand_selection(np.array([[1, 3], [1, 3]]), [1, 0], pool_start, 4, 8)
    assert tok.tolist() == [[7, 8, 9, 10, 15, 16, 17, 18], [4, 5, 6, 7, 12, 13, 14, 15]]


def test_mla_rows_use_their_own_sequence():
    r = _rng(23)
    q = r.standard_normal((2, 2, 8))
    kv = r.standard_normal((2, 20, 8))
    ids = np.array([[1, 5, 9], [1, 5, 9]])
    both, _ = O.sparse_mla_decode(q, kv, [1, 0], ids, 0.4)
    only1, _ = O.sparse_mla_decode(q[:1], kv[1:], [0], ids[:1], 0.4)
    only0, _ = O.sparse_mla_decode(q[1:], kv[:1], [0], ids[:1], 0.4)
    np.testing.assert_array_equal(both[0], only1[0])
    np.testing.assert_array_equal(both[1], only0[0])


def test_expand_id_naming_no_pool_gives_sentinel():
    pool_start = np.array([[2, 6, -1, -1]])
    tok = O.expand_selection(np.array([[1, 2, -1]]), [0], pool_start, 4, 14)
    assert tok.tolist() == [[6, 7, 8, 9] + [-1] * 10]


# ------------------------------------------------------------------ paged / fp8 latent (R14, R15)
def test_fp8_e4m3_decode_matches_torch_and_closed_forms():
    codes = np.arange(256, dtype=np.uint8)
    got = O.fp8_e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert ((got == ref) | (np.isnan(got) & np.isnan(ref))).all()
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x07] == 7 * 2.0 ** -9
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and np.signbit(got[0x80]) and got[0x80] == 0


def _paged_case(fp8: bool, seed: int = 5):
    rng = np.random.default_rng(seed)
    B, T, Dl, Hm, W, ps = 2, 96, 64, 4, 40, 16
    kv = torch.from_numpy(rng.standard_normal((B, T, Dl)).astype(np.float32)).to(torch.bfloat16)
    q = torch.from_numpy(rng.standard_normal((3, Hm, Dl)).astype(np.float32)).to(torch.bfloat16)
    row_seq = np.array([1, 0, 1], np.int32)
    tok = synth.random_token_ids(3, W, [T, T], row_seq.tolist(), seed=seed, hole_frac=0.1).numpy()
    return kv, q, row_seq, tok, synth.paged_latent(kv, ps, seed, fp8=fp8), ps


def test_paged_latent_equals_contiguous_cache():
    # bf16 pages behind a shuffled page table give exactly the contiguous cache's attention
    kv, q, row_seq, tok, pg, ps = _paged_case(False)
    o1, l1 = O.sparse_mla_decode(q, kv, row_seq, tok, 0.125)
    o2, l2 = O.sparse_mla_decode_paged(q, pg["kv_pages"], None, pg["block_table"], ps, row_seq, tok, 0.125)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_paged_out_of_range_page_is_an_absent_token():
    kv, q, row_seq, tok, pg, ps = _paged_case(False, seed=6)
    bt = pg["block_table"].clone()
    t0 = int(tok[0][tok[0] >= 0][0])
    bt[row_seq[0], t0 // ps] = pg["num_pages"] + 7            # a table entry past the pages
    tok_far = tok.copy()
    tok_far[1, 0] = bt.shape[1] * ps + 3                      # a token past the table
    o, l = O.sparse_mla_decode_paged(q, pg["kv_pages"], None, bt, ps, row_seq, tok_far, 0.125)
    ref_tok = tok.copy()
    for r in np.flatnonzero(row_seq == row_seq[0]):          # every row of that sequence
        ref_tok[r][(ref_tok[r] >= 0) & (ref_tok[r] // ps == t0 // ps)] = -1
    ref_tok[1, 0] = -1
    ro, rl = O.sparse_mla_decode(q, kv, row_seq, ref_tok, 0.125)
    np.testing.assert_array_equal(o, ro)
    np.testing.assert_array_equal(l, rl)


def test_fp8_paged_latent_is_the_dequantized_cache():
    # fp8 codes times their row scale (decoded here by torch's float8 type, not the
    # oracle's decoder) as a contiguous cache give the same attention
    kv, q, row_seq, tok, pg, ps = _paged_case(True, seed=7)
    deq = (pg["kv_pages"].view(torch.float8_e4m3fn).double() * pg["kv_scale"].double()[..., None])
    B, T, Dl = kv.shape
    dense = deq[pg["block_table"].reshape(-1).long()].reshape(B, T, Dl)
    o1, l1 = O.sparse_mla_decode(q, dense.numpy(), row_seq, tok, 0.125)
    o2, l2 = O.sparse_mla_decode_paged(q, pg["kv_pages"], pg["kv_scale"], pg["block_table"], ps, row_seq, tok,
                                       0.125)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)
    # and the quantisation itself stays within E4M3's half-ulp of the bf16 cache (2^-4 relative)
    err = np.abs(dense.numpy() - kv.double().numpy())
    assert (err <= np.abs(kv.double().numpy()) * 2.0 ** -4 + pg["kv_scale"].max().item() * 2.0 ** -9).all()


# ---------------------------------------------------------------- whole pipeline
def test_tiny_pipeline_matches_loop_twin():
    """The tiny workload (1 x 256 tokens, 5 left-pad, kpool 4, 4 x 32 index heads,
    select_k 8, 4 x 64 MLA, fp32) through compress -> scores -> top-k -> expand ->
    sparse MLA, by the oracle and by tests/brute.py (scalar loops written
    separately from the same definitions), each stage on its own outputs:
    float results agree to 1e-12, integer results exactly."""
    wl = synth.workload("tiny")
    ti, ip, mi = synth.token_inputs(wl), synth.index_params(wl), synth.mla_inputs(wl)
    L = lambda t: t.double().tolist() if hasattr(t, "double") else list(t)
    row_seq, row_pos = [int(x) for x in ip["row_seq"]], [int(x) for x in ip["row_pos"]]

    comp = O.kpool_compress(ti["k"], ti["gate"], ti["valid"], ti["ape"], ti["seq_len"], wl.kp, wl.P_max)
    pools = brute.compress(L(ti["k"]), L(ti["gate"]), ti["valid"].tolist(), L(ti["ape"]),
                           [int(x) for x in ti["seq_len"]], wl.kp)
    assert len(pools[0]) == comp["n_pools"][0] == 62
    for p, (start, ok, key) in enumerate(pools[0]):
        assert comp["pool_start"][0, p] == start and bool(comp["pool_valid"][0, p]) == ok
        assert np.abs(comp["k_pool"][0, p] - np.array(key)).max() <= 1e-12
    assert (comp["pool_start"][0, 62:] == -1).all() and not comp["pool_valid"][0, 62:].any()

    sc = O.index_scores(ip["q"], ip["w"], ip["scale"], comp["k_pool"], comp["pool_start"], comp["pool_valid"],
                        ip["gamma"], ip["beta"], ip["eps"], ip["row_seq"], ip["row_pos"], wl.kp)
    s64, s32 = brute.scores(L(ip["q"]), L(ip["w"]), ip["scale"], pools, L(ip["gamma"]), L(ip["beta"]),
                            ip["eps"], row_seq, row_pos, wl.kp, wl.P_max)
    s64, s32 = np.array(s64), np.array(s32, dtype=np.float32)
    fin = np.isfinite(s64)
    assert fin[0, :62].all() and not fin[0, 62:].any()
    np.testing.assert_array_equal(sc, s32)                       # same fp32 rounding of each score
    assert np.abs(sc[fin].astype(np.float64) - s64[fin]).max() <= 2.0 ** -24 * np.abs(s64[fin]).max()

    ids = O.topk_pools(sc, wl.K)
    ids_b = brute.topk(s32.astype(np.float64).tolist(), wl.K)
    np.testing.assert_array_equal(ids, np.array(ids_b))

    tok = O.expand_selection(ids, ip["row_seq"], comp["pool_start"], wl.kp, wl.W)
    tok_b = brute.expand(ids_b, row_seq, pools, wl.kp, wl.W)
    np.testing.assert_array_equal(tok, np.array(tok_b))

    out, lse = O.sparse_mla_decode(mi["q_lat"], mi["kv"], ip["row_seq"], tok, mi["sm_scale"])
    out_b, lse_b = brute.attend(L(mi["q_lat"]), L(mi["kv"]), row_seq, tok_b, mi["sm_scale"])
    assert np.abs(out - np.array(out_b)).max() <= 1e-12
    assert np.abs(lse - np.array(lse_b)).max() <= 1e-12
