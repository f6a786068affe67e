"""CPU oracle for DSA token selection and attention over the selected tokens.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check of the package entry
point and the CPU-baseline leg of the benchmark may import or call this module.
The GPU product path never does, and nothing here is shared with it.

Every step is written in float64 NumPy in the order the method states it, one
output at a time where that is clearest, with no blocking, fusion or reordering.
Results are rounded once, round-to-nearest-even, to the stored output dtype.

Sources (the "GLM-5.3 DSA" API pages):
  [DSA]   page "Module glm5next_dsa" (GLM-5.3-Flash DSA production surface):
          sections "Shape of the pipeline", "Traps carried from Slice 8",
          "Constants" (KERNEL_MAX_KPOOL).
  [TP]    page "Module tp" (GLM-5.3 DSA tensor-parallel shard plan):
          section "Why the indexer is REPLICATED, not sharded".

Readings taken where the pages leave a step open (each is also listed in the
design notes of the repository):
  R1  k_norm is applied to the pooled keys, inside the score step.
  R2  LayerNorm epsilon is an argument (1e-5 in the workloads), variance biased.
  R3  ape is [kpool, D], one row per slot; gate is per token and channel.
  R4  w is [Q, H] (one weight per query row and head).
  R5  A pool is a candidate for row q iff it is valid and its last token is at
      or before the row's own position (pool_start + kpool - 1 <= row_pos[q]).
  R6  "Candidate validity" is carried as -inf in the score tensor.
  R7  The selected list is ordered by (score descending, pool index ascending);
      rows with fewer candidates than select_k are padded with -1.  +0 and -0 tie.
  R8  Expansion is pool-major in selection order, slots ascending; token ids
      are absolute positions in the sequence's row; every column past
      select_k*kpool is -1, and so are the slots of a selected id that names
      no pool (pool_start = -1).
  R9  A pool that contains an invalid token (a hole) is not valid; the anchor is
      still the first valid token.
  R10 The sparse attention attends to the listed token ids only (entries -1 are
      skipped); with none it returns 0 and lse = -inf.  The softmax scale is an
      argument.
  R11 Pools p >= n_pools (and every pool of a sequence with no valid token) are
      written as k_pool = 0, pool_start = -1, pool_valid = 0.
  R12 A sequence with no valid token has no pools; its first_valid is reported
      as its length.
  R13 (workload, not arithmetic) The prefill chunk is the last 4096 tokens of
      its sequence, and exact score ties come from pooled keys drawn on the 1/8
      grid from a small codebook with q on the same grid.
  R14 Paged latent cache (the page names a paged decode and an fp8 variant of
      it only by file name): physical pages [num_pages, page_size, Dl]; a page
      table [B, max_pages] maps page j of sequence b to a physical page, so
      token t of sequence b is row t % page_size of page
      block_table[b, t // page_size].  A token whose page index or table entry
      is out of range counts as absent (like -1).
  R15 fp8 latent cache: OCP FP8 E4M3 codes (1 sign, 4 exponent bits with bias
      7, 3 mantissa bits, subnormals, no infinities, S.1111.111 = NaN) and one
      fp32 scale per token row; the latent value is decode(code) * scale.
"""
from __future__ import annotations

import numpy as np

# [DSA] "Constants", KERNEL_MAX_KPOOL: the most pool slots the reference
# compression kernel holds.  Larger values are refused, never truncated.
MAX_KPOOL = 8


# --------------------------------------------------------------------------
# rounding of a float64 result to its stored dtype
# --------------------------------------------------------------------------
def round_f32(x: np.ndarray) -> np.ndarray:
    """float64 -> float32, round-to-nearest-even (one rounding)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bfloat16 value (RNE, one rounding), returned as float32.

    bfloat16 keeps 8 significant bits.  With x = m * 2**e (0.5 <= |m| < 1), the
    spacing of bf16 values around x is 2**(e-8); x / spacing is exact in
    float64 and np.rint rounds half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    _, e = np.frexp(x[nz])
    q = np.ldexp(1.0, np.maximum(e - 8, -133))   # bf16 subnormal spacing is 2**-133
    out[nz] = np.rint(x[nz] / q) * q
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out.astype(np.float32)


def f64(t) -> np.ndarray:
    """Any tensor/array (fp32, bf16, int) -> exact float64 NumPy copy."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            return t.detach().to(torch.float64).cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t, dtype=np.float64)


def _i(t) -> np.ndarray:
    try:
        import torch
        if isinstance(t, torch.Tensor):
            return t.detach().cpu().numpy().astype(np.int64)
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t).astype(np.int64)


# --------------------------------------------------------------------------
# kpool_compress   [DSA] "Shape of the pipeline" (k, gate, valid, ape ->
# pool keys / indices / valid) and "Traps": softmax over the pool-slot axis per
# channel; pooling anchored at the first valid token; a pool counts only if
# every slot is valid (a trailing partial pool is not a pool); kpool <= 8.
# --------------------------------------------------------------------------
def anchor(valid_row: np.ndarray, T_b: int, kp: int) -> tuple[int, int]:
    """(first valid token f_b, number of whole pools after it).

    f_b is the first valid token among the first T_b; with no valid token the
    sequence has no pools (f_b is reported as T_b).  The pools are the whole
    runs of kp tokens starting at f_b that end inside [0, T_b).
    """
    idx = np.flatnonzero(np.asarray(valid_row[:T_b]) != 0)
    if idx.size == 0:
        return T_b, 0
    f_b = int(idx[0])
    return f_b, (T_b - f_b) // kp


def kpool_compress(k, gate, valid, ape, seq_len, kp: int, P_max: int) -> dict:
    """Pooled index keys.

    k, gate: [B, T_max, D]; valid: [B, T_max] (nonzero = valid token);
    ape: [kp, D]; seq_len: [B].  Returns float64 arrays
    k_pool [B, P_max, D], int64 pool_start / n_pools / first_valid, bool pool_valid.

    For pool p of sequence b, slots s = 0..kp-1 are tokens t_s = f_b + p*kp + s.
    Per channel c the slot logits are l_s = gate[b,t_s,c] + ape[s,c]; the weights
    a_s are the softmax of l over s; k_pool[b,p,c] = sum_s a_s * k[b,t_s,c].
    """
    if not (1 <= kp <= MAX_KPOOL):
        raise ValueError(f"kpool {kp} outside [1, {MAX_KPOOL}]")
    k = f64(k); gate = f64(gate); ape = f64(ape)
    valid = _i(valid); seq_len = _i(seq_len)
    B, T_max, D = k.shape
    if P_max < T_max // kp:
        raise ValueError("P_max smaller than T_max // kpool")
    k_pool = np.zeros((B, P_max, D))
    pool_start = np.full((B, P_max), -1, dtype=np.int64)
    pool_valid = np.zeros((B, P_max), dtype=bool)
    n_pools = np.zeros(B, dtype=np.int64)
    first_valid = np.zeros(B, dtype=np.int64)
    for b in range(B):
        T_b = int(seq_len[b])
        f_b, n = anchor(valid[b], T_b, kp)
        first_valid[b] = f_b
        n_pools[b] = n
        for p0 in range(0, n, 8192):                   # pools in chunks (memory only)
            p = np.arange(p0, min(n, p0 + 8192))
            t = f_b + p[:, None] * kp + np.arange(kp)[None, :]   # [np, kp] slot tokens
            logits = gate[b][t] + ape[None, :, :]       # [np, kp, D]
            m = logits.max(axis=1, keepdims=True)       # per pool and channel
            e = np.exp(logits - m)
            a = e / e.sum(axis=1, keepdims=True)        # softmax over the slot axis
            k_pool[b, p, :] = (a * k[b][t]).sum(axis=1)
            pool_start[b, p] = t[:, 0]
            pool_valid[b, p] = np.all(valid[b][t] != 0, axis=1)
    return dict(k_pool=k_pool, pool_start=pool_start, pool_valid=pool_valid,
                n_pools=n_pools, first_valid=first_valid)


# --------------------------------------------------------------------------
# index_scores   [DSA] "Shape of the pipeline" (-> [Q, P] scores + candidate
# validity) and "Traps" (k_norm is nn.LayerNorm: mean-subtracting, with bias);
# [TP] "Why the indexer is REPLICATED": the score is a plain sum over heads of
# weights[h] * relu(scale * dot).
# --------------------------------------------------------------------------
def layer_norm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float) -> np.ndarray:
    """LayerNorm over the last axis with biased variance, scale gamma and bias beta."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * gamma + beta


def candidates(pool_start_b, pool_valid_b, kp: int, row_pos: int) -> np.ndarray:
    """Pools row q may select: valid, and ending at or before the row's position."""
    return np.asarray(pool_valid_b, dtype=bool) & (np.asarray(pool_start_b) + kp - 1 <= row_pos)


def index_scores(q, w, scale: float, k_pool, pool_start, pool_valid, gamma, beta, eps: float,
                 row_seq, row_pos, kp: int, rows=None) -> np.ndarray:
    """scores[q, p] = sum_h w[q,h] * max(0, scale * <q[q,h,:], LN(k_pool[b,p,:])>)
    for candidate pools, -inf otherwise; b = row_seq[q].  Returns float32 [len(rows), P_max].
    """
    q = f64(q); w = f64(w); k_pool = f64(k_pool); gamma = f64(gamma); beta = f64(beta)
    pool_start = _i(pool_start); pool_valid = _i(pool_valid)
    row_seq = _i(row_seq); row_pos = _i(row_pos)
    Q = q.shape[0]
    rows = range(Q) if rows is None else list(rows)
    P_max = k_pool.shape[1]
    out = np.empty((len(rows), P_max), dtype=np.float32)
    normed = {}
    for i, r in enumerate(rows):
        b = int(row_seq[r])
        if b not in normed:
            normed[b] = layer_norm(k_pool[b], gamma, beta, eps)     # [P_max, D]
        kn = normed[b]
        dots = kn @ q[r].T                                         # [P_max, H]
        s = (w[r][None, :] * np.maximum(0.0, scale * dots)).sum(axis=1)
        cand = candidates(pool_start[b], pool_valid[b], kp, int(row_pos[r]))
        out[i] = np.where(cand, round_f32(s), np.float32(-np.inf))
    return out


# --------------------------------------------------------------------------
# topk_pools   [DSA] "Shape of the pipeline" (-> [Q, select_k] pool ids);
# [TP] "Why the indexer is REPLICATED": deterministic tiebreak, higher score
# first, then the smaller pool index.
# --------------------------------------------------------------------------
def topk_pools(scores, K: int) -> np.ndarray:
    """pool_ids[q, j] = j-th candidate of row q in (score desc, index asc) order,
    -1 when the row has fewer than K candidates.  Scores are compared as IEEE
    values (so +0 == -0); -inf marks a non-candidate; NaN is not allowed."""
    s = np.asarray(scores, dtype=np.float32)
    if np.isnan(s).any():
        raise ValueError("NaN score")
    Q, P = s.shape
    out = np.full((Q, K), -1, dtype=np.int32)
    for r in range(Q):
        cand = np.flatnonzero(s[r] != -np.inf)
        vals = s[r, cand].astype(np.float64)
        vals = np.where(vals == 0.0, 0.0, vals)              # -0 ties with +0
        order = np.lexsort((cand, -vals))                    # primary: -score; then index
        take = cand[order[:K]]
        out[r, :take.size] = take
    return out


# --------------------------------------------------------------------------
# expand_selection   [DSA] "Shape of the pipeline" (-> [Q, out_width] token
# ids, -1 = invalid) and "Traps": the -1 sentinel destination is fully written.
# --------------------------------------------------------------------------
def expand_selection(pool_ids, row_seq, pool_start, kp: int, W: int) -> np.ndarray:
    pool_ids = _i(pool_ids); row_seq = _i(row_seq); pool_start = _i(pool_start)
    Q, K = pool_ids.shape
    if W < K * kp:
        raise ValueError("out_width smaller than select_k * kpool")
    tok = np.full((Q, W), -1, dtype=np.int32)
    for r in range(Q):
        b = int(row_seq[r])
        for j in np.flatnonzero(pool_ids[r] >= 0):
            p = pool_ids[r, j]
            if pool_start[b, p] < 0:                # an id that names no pool is invalid
                continue
            tok[r, j * kp:(j + 1) * kp] = pool_start[b, p] + np.arange(kp)
    return tok


# --------------------------------------------------------------------------
# sparse MLA decode   [DSA] "Shape of the pipeline" (NoPE MLA restricted to
# the selected tokens) and "Traps" (NoPE: the rotary slice is zero-width);
# [TP] "Traps": kv_a_proj_with_mqa yields one shared latent per token, no head
# axis -- so the cache is [B, T, Dl] and, absorbed, keys = values = latent.
# --------------------------------------------------------------------------
def sparse_mla_decode(q_lat, kv, row_seq, token_ids, sm_scale: float, rows=None):
    """out[q,h,:] = sum_j softmax_j(sm_scale * <q_lat[q,h], kv[b,j]>) kv[b,j]
    over the listed ids j >= 0 of row q (b = row_seq[q]); lse[q,h] = log-sum-exp
    of those logits.  Returns float64 (out [R, Hm, Dl], lse [R, Hm])."""
    q_lat = f64(q_lat); row_seq = _i(row_seq); token_ids = _i(token_ids)
    Q, Hm, Dl = q_lat.shape
    rows = range(Q) if rows is None else list(rows)
    out = np.zeros((len(rows), Hm, Dl))
    lse = np.full((len(rows), Hm), -np.inf)
    for i, r in enumerate(rows):
        b = int(row_seq[r])
        ids = token_ids[r][token_ids[r] >= 0]
        if ids.size == 0:
            continue
        V = f64(kv[b, ids])                                   # [n, Dl] gathered latents
        logits = sm_scale * (q_lat[r] @ V.T)                  # [Hm, n]
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        l = e.sum(axis=1, keepdims=True)
        out[i] = (e @ V) / l
        lse[i] = (m + np.log(l))[:, 0]
    return out, lse


# --------------------------------------------------------------------------
# paged and fp8 latent cache (readings R14, R15): the attention above over a
# latent cache stored in pages, optionally as fp8 E4M3 codes with a scale per
# token row.  [DSA] module list: "attend", the launcher of the selected-index
# NoPE MLA *paged* decode; "Constants": mla_paged_decode{,_fp8}.
# --------------------------------------------------------------------------
def fp8_e4m3_decode(codes) -> np.ndarray:
    """OCP FP8 E4M3 code -> exact float64: sign * 2^(e-7) * (1 + m/8) for
    e = 1..15 (except e = 15, m = 7: NaN), sign * 2^-6 * m/8 for e = 0."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def paged_latent_rows(kv_pages, kv_scale=None) -> np.ndarray:
    """Physical latent rows [num_pages * page_size, Dl] in float64: bf16/fp32
    pages widened exactly, or fp8 E4M3 codes (uint8) decoded and multiplied by
    their row's scale (kv_scale [num_pages, page_size])."""
    if kv_scale is None:
        kv = f64(kv_pages)
        return kv.reshape(-1, kv.shape[-1])
    codes = np.asarray(kv_pages.numpy() if hasattr(kv_pages, "numpy") else kv_pages, dtype=np.uint8)
    vals = fp8_e4m3_decode(codes).reshape(-1, codes.shape[-1])
    return vals * f64(kv_scale).reshape(-1, 1)


def paged_token_rows(token_ids, row_seq, block_table, page_size: int, num_pages: int) -> np.ndarray:
    """Physical row of each listed token (R14): -1 for -1 entries and for tokens
    whose page index or page-table entry is out of range."""
    tok = _i(token_ids); row_seq = _i(row_seq); bt = _i(block_table)
    max_pages = bt.shape[1]
    out = np.full(tok.shape, -1, dtype=np.int64)
    for r in range(tok.shape[0]):
        b = int(row_seq[r])
        for c in range(tok.shape[1]):
            t = int(tok[r, c])
            if t < 0 or t // page_size >= max_pages:
                continue
            pg = int(bt[b, t // page_size])
            if 0 <= pg < num_pages:
                out[r, c] = pg * page_size + t % page_size
    return out


def sparse_mla_decode_paged(q_lat, kv_pages, kv_scale, block_table, page_size: int, row_seq, token_ids,
                            sm_scale: float, rows=None):
    """sparse_mla_decode over a paged (optionally fp8) latent cache: each listed
    token is resolved to its physical row (R14), the rows are dequantized (R15),
    and the same softmax attention is taken over them."""
    num_pages = int(np.asarray(kv_pages.shape)[0])
    phys = paged_token_rows(token_ids, row_seq, block_table, page_size, num_pages)
    flat = paged_latent_rows(kv_pages, kv_scale)[None]         # one "sequence" holding every row
    return sparse_mla_decode(q_lat, flat, np.zeros_like(_i(row_seq)), phys, sm_scale, rows=rows)
