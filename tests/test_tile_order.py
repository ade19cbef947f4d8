"""The GEMM's renumbering of workgroups to tiles (the XCD-aware order of k_gemm_nt's
tile_xy) is a bijection on every grid shape: every tile computed exactly once.  The index
arithmetic is restated here as the kernel does it, on the host."""

import pytest


def tile_xy(L, gx, gy):
    n = gx * gy
    if n % 32 == 0 and gx % 4 == 0 and 32 % gx == 0:
        L = (L & 7) * (n >> 3) + (L >> 3)
        per, cols = n >> 3, gx // 4
        xcd, w = L // per, L % per
        return (xcd % cols) * 4 + w % 4, (xcd // cols) * (per // 4) + w // 4
    if gx % 8 == 0:
        xcd, idx, cx = L & 7, L >> 3, gx >> 3
        bw = next((d for d in range(8, 1, -1) if cx % d == 0), 1)
        band, r = idx // (bw * gy), idx % (bw * gy)
        return xcd * cx + band * bw + r % bw, r // bw
    if n % 8 == 0:
        L = (L & 7) * (n >> 3) + (L >> 3)
    return L % gx, L // gx


@pytest.mark.parametrize("gx", list(range(1, 41)) + [48, 56, 64, 112, 120, 224])
def test_tile_order_is_a_bijection(gx):
    for gy in list(range(1, 34)) + [64, 128]:
        seen = set()
        for L in range(gx * gy):
            tx, ty = tile_xy(L, gx, gy)
            assert 0 <= tx < gx and 0 <= ty < gy, (gx, gy, L, tx, ty)
            seen.add((tx, ty))
        assert len(seen) == gx * gy, (gx, gy)


def test_wide_products_send_each_weight_block_to_one_xcd():
    """28672 x 8192 at M = 2048 (112 x 8 tiles): the workgroups dealt to one XCD (L % 8)
    cover feature columns no other XCD touches."""
    gx, gy = 112, 8
    cols = {x: set() for x in range(8)}
    for L in range(gx * gy):
        cols[L % 8].add(tile_xy(L, gx, gy)[0])
    for a in range(8):
        assert len(cols[a]) == gx // 8
        for b in range(a + 1, 8):
            assert not cols[a] & cols[b]
