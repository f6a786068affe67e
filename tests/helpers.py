"""Shared helpers of the GPU parity tests: input preparation and tolerance checks.

Inputs come from dsa_decode_amd.synth (seeded) and, for later stages, from the
oracle's own earlier stages; nothing here reads a GPU result back into the
oracle.
"""
from __future__ import annotations

import numpy as np
import torch

from dsa_decode_amd.layout import tile_pool_cache, untile_pool_cache  # noqa: F401

from oracle import dsa_oracle as O


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().cuda()


def act_from_f64(x: np.ndarray, dtype) -> torch.Tensor:
    """Oracle float64 values -> stored activation dtype (one RNE rounding)."""
    if dtype == torch.bfloat16:
        return torch.from_numpy(O.round_bf16(x)).to(torch.bfloat16)
    return torch.from_numpy(O.round_f32(x))


def pool_cache_from_oracle(comp: dict, dtype) -> dict:
    """The oracle's compress outputs in the stored layout of the pool cache."""
    return dict(k_pool=act_from_f64(comp["k_pool"], dtype),
                pool_start=torch.from_numpy(comp["pool_start"].astype(np.int32)),
                pool_valid=torch.from_numpy(comp["pool_valid"].astype(np.uint8)),
                n_pools=torch.from_numpy(comp["n_pools"].astype(np.int32)),
                first_valid=torch.from_numpy(comp["first_valid"].astype(np.int32)))


def bf16_spacing(x: np.ndarray) -> np.ndarray:
    """Distance between adjacent bf16 values around |x| (the ulp used for 1-ulp checks)."""
    ax = np.abs(np.asarray(x, np.float64))
    _, e = np.frexp(np.where(ax > 0, ax, 1.0))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def assert_compress_close(got_kpool: torch.Tensor, ref_f64: np.ndarray, absk_pool_f64: np.ndarray,
                          dtype) -> None:
    """|g - o| <= s + 1e-5 * sum_s a_s |k_s|, with s one bf16 spacing of o for bf16
    outputs (the stored rounding) and 0 for fp32; the second term is the fp32
    forward-error floor for pools whose weighted sum cancels.  bf16 outputs
    must also be >= 98% bit-equal to the oracle rounded once (RNE)."""
    g = got_kpool.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - ref_f64)
    tol = 1e-5 * absk_pool_f64 + 1e-30
    if dtype == torch.bfloat16:
        tol = tol + bf16_spacing(ref_f64)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{bad.sum()} values out of tolerance; first at {tuple(i)}: got {g[tuple(i)]}, "
                             f"oracle {ref_f64[tuple(i)]}, sum a|k| {absk_pool_f64[tuple(i)]}")
    if dtype == torch.bfloat16:
        eq = np.mean(g == O.round_bf16(ref_f64).astype(np.float64))
        assert eq >= 0.98, f"only {eq:.4f} bit-equal to the RNE-rounded oracle"


def score_scale(q, w, scale, k_pool, gamma, beta, eps, row_seq, rows) -> np.ndarray:
    """Forward-error scale A[q,p] = sum_h |w| |scale| sum_c |q * kn| per (row, pool)."""
    qf = O.f64(q); wf = O.f64(w); kp = O.f64(k_pool); g = O.f64(gamma); b = O.f64(beta)
    rs = np.asarray(row_seq.cpu() if isinstance(row_seq, torch.Tensor) else row_seq).astype(np.int64)
    out = []
    cache = {}
    for r in rows:
        bb = int(rs[r])
        if bb not in cache:
            cache[bb] = np.abs(O.layer_norm(kp[bb], g, b, eps))
        akn = cache[bb]
        out.append((np.abs(akn) @ np.abs(qf[r]).T * np.abs(scale) * np.abs(wf[r])[None]).sum(axis=1))
    return np.stack(out)


def assert_scores_close(got: np.ndarray, ref: np.ndarray, A: np.ndarray) -> None:
    """Candidates: |g - o| <= 1e-3 |o| + 1e-5 A; non-candidates: both exactly -inf."""
    ninf_g = got == -np.inf
    ninf_r = ref == -np.inf
    assert (ninf_g == ninf_r).all(), f"candidate mask differs at {np.argwhere(ninf_g != ninf_r)[:5]}"
    m = ~ninf_r
    err = np.abs(got[m].astype(np.float64) - ref[m].astype(np.float64))
    tol = 1e-3 * np.abs(ref[m].astype(np.float64)) + 1e-5 * A[m]
    assert (err <= tol).all(), f"max err/tol {np.max(err / tol)} ({(err > tol).sum()} bad)"


def assert_topk_property(scores: np.ndarray, ids: np.ndarray, K: int) -> None:
    """Checks a selection against its own score rows (valid at any size):
    ids are the candidates in (score desc, index asc) order, the first
    min(K, #candidates) of them, -1 padded."""
    for r in range(scores.shape[0]):
        s = scores[r]
        cand = np.flatnonzero(s != -np.inf)
        n = min(K, cand.size)
        row = ids[r]
        assert (row[n:] == -1).all()
        sel = row[:n]
        assert (sel >= 0).all() and len(np.unique(sel)) == n
        v = s[sel].astype(np.float64)
        v = np.where(v == 0, 0.0, v)
        # order: score desc, index asc
        ok = (v[:-1] > v[1:]) | ((v[:-1] == v[1:]) & (sel[:-1] < sel[1:]))
        assert ok.all(), f"row {r}: order broken"
        if n < cand.size:
            rest = np.setdiff1d(cand, sel)
            rv = np.where(s[rest] == 0, 0.0, s[rest].astype(np.float64))
            last_v, last_i = v[-1], sel[-1]
            assert ((rv < last_v) | ((rv == last_v) & (rest > last_i))).all(), f"row {r}: a better pool left out"
