"""Seeded synthetic inputs for the DSA select + attend path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no pooling, no normalisation, no scoring, no selection).
Both the CPU oracle and the GPU path are fed from it.

Workloads (all synthetic, sizes from the DSA decode/prefill shapes):

* ``tiny``     fp32: 1 sequence of 256 tokens, 5 left-pad invalid tokens, kpool 4,
               4 index heads x 32, select_k 8 pools, 1 query row, MLA 4 heads x 64.
* ``decode``   bf16: 1 sequence of 8192 tokens, kpool 4, 32 index heads x 128,
               select_k 512 pools, MLA 64 heads over a 512-wide latent.
* ``batched``  bf16: 32 sequences, lengths ~U{16384..65536}, left pad ~U{0..31}.
* ``long``     bf16: 4 sequences of 262144 tokens (65536 pools each).
* ``prefill``  bf16: 4096 query rows at the end of a 131072-token sequence, causal
               pool validity per row; q and the pooled keys on a 1/8 grid, keys drawn
               from a 256-row codebook so that exact score ties straddle the cut.

Value distributions: k, q, gate ~ N(0,1); ape ~ N(0, 0.1); w[q,h] ~ U(0,1)/H;
scale = 1/sqrt(D); LayerNorm gamma ~ 1 + N(0, 0.02), beta ~ N(0, 0.02);
q_lat, kv ~ N(0,1); sm_scale = 1/sqrt(Dl).  The second argument of N is a
standard deviation.  Values are drawn in fp32 and rounded once (RNE) to the
activation dtype; both sides read the same bits.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np
import torch

WORKLOADS = ("tiny", "decode", "batched", "long", "prefill")


@dataclass
class Workload:
    name: str
    seed: int
    B: int
    T_max: int
    seq_len: list
    pad: list
    kp: int
    H: int
    D: int
    K: int
    Hm: int
    Dl: int
    dtype: str                      # "f32" or "bf16" (activations)
    Q: int = 0                      # query rows (filled in by workload())
    prefill: bool = False
    extra: dict = field(default_factory=dict)

    @property
    def P_max(self) -> int:
        return self.T_max // self.kp

    @property
    def W(self) -> int:
        return self.K * self.kp

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


def workload(name: str, *, seed: int | None = None) -> Workload:
    """The geometry of one named workload (lengths drawn from its seed)."""
    idx = WORKLOADS.index(name)
    seed = 1000 + idx if seed is None else seed
    if name == "tiny":
        wl = Workload(name, seed, 1, 256, [256], [5], 4, 4, 32, 8, 4, 64, "f32")
    elif name == "decode":
        wl = Workload(name, seed, 1, 8192, [8192], [0], 4, 32, 128, 512, 64, 512, "bf16")
    elif name == "batched":
        rng = np.random.Generator(np.random.PCG64(seed))
        lens = rng.integers(16384, 65536, size=32, endpoint=True).tolist()
        pads = rng.integers(0, 31, size=32, endpoint=True).tolist()
        wl = Workload(name, seed, 32, max(lens), lens, pads, 4, 32, 128, 512, 64, 512, "bf16")
    elif name == "long":
        wl = Workload(name, seed, 4, 262144, [262144] * 4, [0] * 4, 4, 32, 128, 512, 64, 512, "bf16")
    elif name == "prefill":
        wl = Workload(name, seed, 1, 131072, [131072], [0], 4, 32, 128, 512, 64, 512, "bf16",
                      prefill=True)
    else:  # pragma: no cover
        raise KeyError(name)
    wl.Q = 4096 if wl.prefill else wl.B
    return wl


def _rng(seed: int, stream: int) -> np.random.Generator:
    # one independent PCG64 stream per tensor, so that drawing one tensor never
    # shifts another's values
    return np.random.Generator(np.random.PCG64([seed, stream]))


def _normal(seed, stream, shape, std=1.0, mean=0.0) -> np.ndarray:
    x = _rng(seed, stream).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def _act(x: np.ndarray, wl: Workload) -> torch.Tensor:
    """fp32 draw -> activation dtype (one RNE rounding for bf16)."""
    return torch.from_numpy(x).to(wl.torch_dtype)


def token_inputs(wl: Workload, *, with_gate: bool = True) -> dict:
    """Token-level inputs of the pooled-key compression.

    k, gate: [B, T_max, D] activation dtype; valid: [B, T_max] uint8;
    ape: [kp, D] fp32; seq_len: [B] int32.  Tokens at or beyond seq_len[b] are
    invalid and hold random values (they must not influence anything).
    """
    B, T, D = wl.B, wl.T_max, wl.D
    k = _act(_normal(wl.seed, 1, (B, T, D)), wl)
    gate = _act(_normal(wl.seed, 2, (B, T, D)), wl) if with_gate else None
    valid = np.zeros((B, T), dtype=np.uint8)
    for b in range(B):
        valid[b, wl.pad[b]:wl.seq_len[b]] = 1
    ape = torch.from_numpy(_normal(wl.seed, 3, (wl.kp, D), std=0.1))
    return dict(k=k, gate=gate, valid=torch.from_numpy(valid), ape=ape,
                seq_len=torch.tensor(wl.seq_len, dtype=torch.int32))


def index_params(wl: Workload) -> dict:
    """Query-side inputs of the index scores.

    q: [Q, H, D] activation dtype; w: [Q, H] fp32 ~ U(0,1)/H; gamma, beta: [D] fp32;
    row_seq, row_pos: [Q] int32 (decode: one row per sequence at its last token;
    prefill: the last Q tokens of sequence 0).
    """
    Q, H, D = wl.Q, wl.H, wl.D
    qf = _normal(wl.seed, 4, (Q, H, D))
    if wl.prefill:
        qf = np.clip(np.round(qf * 8.0) / 8.0, -4.0, 4.0).astype(np.float32)
    q = _act(qf, wl)
    w = torch.from_numpy((_rng(wl.seed, 5).random(size=(Q, H), dtype=np.float32)
                          / np.float32(H)).astype(np.float32))
    gamma = torch.from_numpy(_normal(wl.seed, 6, (D,), std=0.02, mean=1.0))
    beta = torch.from_numpy(_normal(wl.seed, 7, (D,), std=0.02))
    if wl.prefill:
        T = wl.seq_len[0]
        row_pos = np.arange(T - Q, T, dtype=np.int32)
        row_seq = np.zeros(Q, dtype=np.int32)
    else:
        row_pos = np.array([wl.seq_len[b] - 1 for b in range(wl.B)], dtype=np.int32)
        row_seq = np.arange(wl.B, dtype=np.int32)
    return dict(q=q, w=w, scale=1.0 / math.sqrt(D), gamma=gamma, beta=beta, eps=1e-5,
                row_seq=torch.from_numpy(row_seq), row_pos=torch.from_numpy(row_pos))


def codebook_keys(wl: Workload, n_codes: int = 256) -> torch.Tensor:
    """Pooled keys drawn from a small codebook on the 1/8 grid: [B, P_max, D].

    Each pool row is one of ``n_codes`` fixed vectors, so equal rows (and hence
    exactly equal scores) recur about P_max/n_codes times per row of scores.
    """
    code = np.clip(np.round(_normal(wl.seed, 8, (n_codes, wl.D)) * 8.0) / 8.0, -4.0, 4.0)
    pick = _rng(wl.seed, 9).integers(0, n_codes, size=(wl.B, wl.P_max))
    return _act(code.astype(np.float32)[pick], wl)


def mla_inputs(wl: Workload, *, kv_seed_stream: int = 10) -> dict:
    """q_lat: [Q, Hm, Dl]; kv: [B, T_max, Dl] (activation dtype); sm_scale = 1/sqrt(Dl)."""
    q_lat = _act(_normal(wl.seed, 11, (wl.Q, wl.Hm, wl.Dl)), wl)
    kv = _act(_normal(wl.seed, kv_seed_stream, (wl.B, wl.T_max, wl.Dl)), wl)
    return dict(q_lat=q_lat, kv=kv, sm_scale=1.0 / math.sqrt(wl.Dl))


def random_scores(Q: int, P: int, seed: int, *, tie_levels: int = 0, neg_inf_frac: float = 0.0,
                  signed_zeros: bool = False) -> torch.Tensor:
    """A synthetic fp32 score tensor [Q, P] for exercising the selection alone.

    tie_levels > 0 draws every score from that many distinct values (forced ties);
    neg_inf_frac marks that fraction of entries as non-candidates (-inf);
    signed_zeros puts +0.0 and -0.0 among the values.
    """
    rng = _rng(seed, 20)
    if tie_levels > 0:
        levels = rng.standard_normal(tie_levels).astype(np.float32)
        s = levels[rng.integers(0, tie_levels, size=(Q, P))]
    else:
        s = rng.standard_normal((Q, P)).astype(np.float32)
    if signed_zeros:
        z = rng.random((Q, P)) < 0.05
        sign = rng.random((Q, P)) < 0.5
        s[z & sign] = np.float32(0.0)
        s[z & ~sign] = np.float32(-0.0)
    if neg_inf_frac > 0:
        s[rng.random((Q, P)) < neg_inf_frac] = -np.inf
    return torch.from_numpy(np.ascontiguousarray(s, dtype=np.float32))


def random_token_ids(Q: int, W: int, n_tokens: list, row_seq: list, seed: int, *,
                     hole_frac: float = 0.0) -> torch.Tensor:
    """Unique random token ids per row (drawn from [0, n_tokens[row_seq[q]])), -1 holes."""
    rng = _rng(seed, 21)
    out = np.full((Q, W), -1, dtype=np.int32)
    for qi in range(Q):
        n = n_tokens[row_seq[qi]]
        take = min(W, n)
        ids = rng.choice(n, size=take, replace=False).astype(np.int32)
        if hole_frac > 0:
            ids[rng.random(take) < hole_frac] = -1
        out[qi, :take] = ids
    return torch.from_numpy(out)


def paged_latent(kv: torch.Tensor, page_size: int, seed: int, *, fp8: bool = False,
                 spare_pages: int = 3) -> dict:
    """A latent cache [B, T_max, Dl] laid out in pages for the paged decode.

    Returns kv_pages [num_pages, page_size, Dl] (bf16, or uint8 OCP FP8 E4M3
    codes when fp8), kv_scale [num_pages, page_size] fp32 (fp8 only: the row's
    max |value| / 448, so codes span the format's range) and block_table
    [B, T_max / page_size] int32: page j of sequence b sits at a random
    physical page (a seeded permutation, with spare_pages unused pages mixed in).
    """
    B, T, Dl = kv.shape
    assert T % page_size == 0
    per = T // page_size
    num_pages = B * per + spare_pages
    perm = _rng(seed, 31).permutation(num_pages)[: B * per].astype(np.int32)
    block_table = torch.from_numpy(perm.reshape(B, per).copy())
    rows = kv.reshape(B * per, page_size, Dl)
    if not fp8:
        pages = torch.zeros((num_pages, page_size, Dl), dtype=kv.dtype)
        pages[torch.from_numpy(perm.astype(np.int64))] = rows
        return dict(kv_pages=pages, kv_scale=None, block_table=block_table, num_pages=num_pages)
    x = rows.float()
    amax = x.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)
    scale = (amax / 448.0).float()
    codes = (x / scale).to(torch.float8_e4m3fn).view(torch.uint8)
    pages = torch.zeros((num_pages, page_size, Dl), dtype=torch.uint8)
    sc = torch.ones((num_pages, page_size), dtype=torch.float32)
    idx = torch.from_numpy(perm.astype(np.int64))
    pages[idx] = codes
    sc[idx] = scale[..., 0]
    return dict(kv_pages=pages, kv_scale=sc, block_table=block_table, num_pages=num_pages)
