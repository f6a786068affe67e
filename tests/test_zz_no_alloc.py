"""dsa_sparse_mla_decode_noalloc (the partials in the library's fixed per-GPU
buffer) against dsa_sparse_mla_decode with a caller workspace: the same
kernels, so the outputs must be the same bits.  Two calls in a row on the one
buffer, the second with a smaller input (fewer rows, fewer ids, fewer heads),
then a call that needs more than the buffer holds, refused before any launch."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from dsa_decode_amd import _lib, ops
from tests.helpers import dev

pytestmark = pytest.mark.gpu


def _inputs(Q, Hm, W, B, T, seed):
    rng = np.random.default_rng(seed)
    q_lat = torch.from_numpy(rng.standard_normal((Q, Hm, 512)).astype(np.float32)).to(torch.bfloat16)
    kv = torch.from_numpy(rng.standard_normal((B, T, 512)).astype(np.float32)).to(torch.bfloat16)
    row_seq = rng.integers(0, B, Q).astype(np.int32)
    tok = np.stack([rng.permutation(T)[:W] for _ in range(Q)]).astype(np.int32)
    tok[:, ::7] = -1                      # holes in every row
    tok[0, :] = -1                        # a row with no id
    return dev(q_lat), dev(kv), dev(torch.from_numpy(row_seq)), dev(torch.from_numpy(tok))


def _both(q_lat, kv, row_seq, tok, sm_scale):
    Q, Hm, _ = q_lat.shape
    ref_o, ref_l = ops.dsa_sparse_mla_decode(q_lat, kv, row_seq, tok, sm_scale)
    out = torch.full((Q, Hm, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((Q, Hm), float("nan"), dtype=torch.float32, device="cuda")
    ops.dsa_sparse_mla_decode_noalloc(q_lat, kv, row_seq, tok, sm_scale, out, lse)
    torch.cuda.synchronize()
    return ref_o, ref_l, out, lse


def test_noalloc_mla_matches_workspace_entry_point_twice():
    sm = 512 ** -0.5
    # first call: the long-context decode step's shape (4 rows x 2048 ids, 64 heads: 32 splits)
    a = _inputs(4, 64, 2048, 4, 20000, seed=5)
    assert 0 < ops.dsa_sparse_mla_workspace_bytes(4, 64, 512, 2048, ops.DSA_BF16) <= ops.DSA_MLA_SCRATCH_BYTES
    ref_o, ref_l, out, lse = _both(*a, sm)
    assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16))
    assert torch.equal(lse, ref_l)
    # second call on the same buffer, smaller: 2 rows x 700 ids, 32 heads (11 splits)
    b = _inputs(2, 32, 700, 2, 9000, seed=6)
    ref_o, ref_l, out, lse = _both(*b, sm)
    assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16))
    assert torch.equal(lse, ref_l)
    assert torch.isnan(lse[0]).sum() == 0 and (lse[0] == -float("inf")).all()


def test_noalloc_mla_refuses_what_does_not_fit():
    Q, Hm, W = 64, 64, 4096
    need = ops.dsa_sparse_mla_workspace_bytes(Q, Hm, 512, W, ops.DSA_BF16)
    assert need > ops.DSA_MLA_SCRATCH_BYTES
    lib = _lib.load()
    fake = 256  # never dereferenced: the size check comes before any launch
    st = lib.dsa_sparse_mla_decode_noalloc(fake, fake, fake, fake, Q, Hm, 512, 1, 100000, W, 0.04, ops.DSA_BF16,
                                           fake, fake, None)
    assert st == _lib.DSA_ERR_TOO_LARGE
