"""Host-side pool-cache layout helpers against the layout's index formula
(the tile-interleaved cache that dsa_kpool_compress writes and
dsa_index_scores reads, include/dsa.h)."""
import torch

from dsa_decode_amd.layout import pool_cache_pools, tile_pool_cache, untile_pool_cache


def _index(b, p, ch, Pt, D, E):
    return (((b * Pt + (p >> 4)) * (D // E) + ch // E) * 16 + (p & 15)) * E + ch % E


def test_tile_matches_index_formula_and_round_trips():
    for dtype, E in [(torch.bfloat16, 8), (torch.float32, 4)]:
        for B, P, D in [(2, 37, 32), (1, 16, 128), (3, 1, 8 if E == 8 else 4)]:
            x = (torch.arange(B * P * D, dtype=torch.float32).reshape(B, P, D) % 251).to(dtype)
            t = tile_pool_cache(x)
            Pt = (P + 15) // 16
            assert tuple(t.shape) == (B, pool_cache_pools(P), D)
            flat = t.reshape(-1)
            for b in range(B):
                for p in range(P):
                    for ch in range(D):
                        assert flat[_index(b, p, ch, Pt, D, E)] == x[b, p, ch]
            assert torch.equal(untile_pool_cache(t, P), x)
            # padding pools of the last tile are zero
            assert (untile_pool_cache(t, Pt * 16)[:, P:] == 0).all()


def test_a_tile_k_step_is_one_contiguous_kibibyte():
    # bf16, D = 128: lane (kg, ln) of the matrix-core operand for k-step i holds
    # pool ln, channels 8*(kg + 4i) .. +8; those 64 lanes' pieces are elements
    # [512 i, 512 i + 512) of the tile, lane-major
    x = torch.arange(16 * 128, dtype=torch.float32).reshape(1, 16, 128).to(torch.bfloat16)
    t = tile_pool_cache(x).reshape(-1)
    for i in range(4):
        for lane in range(64):
            kg, ln = lane >> 4, lane & 15
            seg = t[512 * i + 8 * lane: 512 * i + 8 * lane + 8]
            assert torch.equal(seg, x[0, ln, 8 * (kg + 4 * i): 8 * (kg + 4 * i) + 8])
