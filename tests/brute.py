"""A second, loop-by-loop implementation of the DSA select+attend pipeline,
used only to pin the oracle on the tiny workload (test infrastructure).

It is written independently of ``oracle/``: plain Python scalars and the
``math`` module, one output element at a time, no NumPy arithmetic, so that a
slip in the oracle's vectorised indexing (a transposed operand, a wrong axis
of the softmax or the LayerNorm, a dropped term) shows up as a disagreement.

Sources: page "Module glm5next_dsa" (GLM-5.3-Flash DSA production surface),
sections "Shape of the pipeline" and "Traps carried from Slice 8"; page
"Module tp", section "Why the indexer is REPLICATED, not sharded" (the score
as a weighted sum of ReLU'd head dots; ordering by score, then pool index).
"""
from __future__ import annotations

import math
import struct


def _f32(x: float) -> float:
    """x rounded to the nearest float32 (ties to even)."""
    return struct.unpack("f", struct.pack("f", x))[0]


def compress(k, gate, valid, ape, seq_len, kp):
    """Pooled keys of every sequence.

    k, gate: nested lists [B][T][D]; valid: [B][T] (0/1); ape: [kp][D].
    Pools start at the first valid token and are whole runs of kp tokens that
    end inside the sequence; each channel's slot weights are the softmax over
    the kp slots of gate + ape.  Returns per sequence a list of pools, each
    (start token, is_valid, key [D]).
    """
    out = []
    for b in range(len(k)):
        T_b = seq_len[b]
        first = None
        for t in range(T_b):
            if valid[b][t]:
                first = t
                break
        pools = []
        if first is not None:
            D = len(k[b][0])
            for p in range((T_b - first) // kp):
                toks = [first + p * kp + s for s in range(kp)]
                key = []
                for c in range(D):
                    logits = [gate[b][t][c] + ape[s][c] for s, t in enumerate(toks)]
                    top = max(logits)
                    ex = [math.exp(v - top) for v in logits]
                    tot = sum(ex)
                    key.append(sum(ex[s] / tot * k[b][t][c] for s, t in enumerate(toks)))
                ok = all(valid[b][t] for t in toks)
                pools.append((toks[0], ok, key))
        out.append(pools)
    return out


def layer_norm_row(x, gamma, beta, eps):
    """One row: subtract the mean, divide by sqrt(biased variance + eps), then
    scale and shift per channel."""
    n = len(x)
    mean = sum(x) / n
    var = sum((v - mean) * (v - mean) for v in x) / n
    inv = 1.0 / math.sqrt(var + eps)
    return [(x[c] - mean) * inv * gamma[c] + beta[c] for c in range(n)]


def scores(q, w, scale, pools, gamma, beta, eps, row_seq, row_pos, kp, P_max):
    """Row r, pool p: sum over heads of w[r][h] * max(0, scale * <q[r][h], LN(key_p)>)
    for a valid pool whose last token is at or before row_pos[r]; -inf for every
    other pool slot up to P_max.  Returns (fp64 scores, the same rounded to fp32)."""
    exact, rounded = [], []
    for r in range(len(q)):
        plist = pools[row_seq[r]]
        row64, row32 = [], []
        for p in range(P_max):
            if p >= len(plist) or not plist[p][1] or plist[p][0] + kp - 1 > row_pos[r]:
                row64.append(-math.inf)
                row32.append(-math.inf)
                continue
            kn = layer_norm_row(plist[p][2], gamma, beta, eps)
            s = 0.0
            for h in range(len(q[r])):
                dot = 0.0
                for c in range(len(kn)):
                    dot += q[r][h][c] * kn[c]
                s += w[r][h] * max(0.0, scale * dot)
            row64.append(s)
            row32.append(_f32(s))
        exact.append(row64)
        rounded.append(row32)
    return exact, rounded


def topk(score_rows, K):
    """Per row: candidates (score > -inf) by higher score first, then smaller
    pool index; the first K, padded with -1.  +0 and -0 compare equal."""
    out = []
    for row in score_rows:
        cand = [(-(v + 0.0), p) for p, v in enumerate(row) if v != -math.inf]
        cand.sort()
        ids = [p for _, p in cand[:K]]
        out.append(ids + [-1] * (K - len(ids)))
    return out


def expand(ids_rows, row_seq, pools, kp, W):
    """Selected pool j of a row -> its kp token ids in columns j*kp .. j*kp+kp-1;
    every other column -1."""
    out = []
    for r, ids in enumerate(ids_rows):
        row = [-1] * W
        plist = pools[row_seq[r]]
        for j, p in enumerate(ids):
            if 0 <= p < len(plist):
                for s in range(kp):
                    row[j * kp + s] = plist[p][0] + s
        out.append(row)
    return out


def attend(q_lat, kv, row_seq, tok_rows, sm_scale):
    """Per row and head: softmax over the listed tokens of sm_scale * <q, kv_t>,
    and the softmax-weighted sum of the same latent rows kv_t (keys = values).
    Returns (out [Q][Hm][Dl], lse [Q][Hm]); a row with no token gives 0, -inf."""
    outs, lses = [], []
    for r in range(len(q_lat)):
        b = row_seq[r]
        toks = [t for t in tok_rows[r] if t >= 0]
        o_r, l_r = [], []
        for h in range(len(q_lat[r])):
            qv = q_lat[r][h]
            Dl = len(qv)
            if not toks:
                o_r.append([0.0] * Dl)
                l_r.append(-math.inf)
                continue
            logits = []
            for t in toks:
                d = 0.0
                for c in range(Dl):
                    d += qv[c] * kv[b][t][c]
                logits.append(sm_scale * d)
            top = max(logits)
            ex = [math.exp(v - top) for v in logits]
            tot = sum(ex)
            o = [0.0] * Dl
            for i, t in enumerate(toks):
                for c in range(Dl):
                    o[c] += ex[i] * kv[b][t][c]
            o_r.append([v / tot for v in o])
            l_r.append(top + math.log(tot))
        outs.append(o_r)
        lses.append(l_r)
    return outs, lses
