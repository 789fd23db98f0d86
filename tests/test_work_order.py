"""Fixed-length work order of the forward kernels (attn_kernels.hpp,
block_to_work, with the order the host's plan() picks in attn_api.cpp),
restated here: every launch index must map to a distinct (batch*head, query
tile) pair, so that each query tile is computed exactly once."""

import itertools

import pytest


def plan_remap(B, H, N, causal, rows=256):
    tiles = -(-N // rows)
    grid = B * H * tiles
    remap = 1 if grid % 8 == 0 else 0
    if remap and causal and tiles < 32 and (B * H) % 8 == 0:
        remap = 2
    return tiles, grid, remap


def block_to_work(L, grid, B, H, n_qtiles, remap):
    if remap == 2:
        hx = (B * H) >> 3
        k = L >> 3
        t = k // hx
        return (L & 7) * hx + (k - t * hx), n_qtiles - 1 - t
    if remap:
        per = grid >> 3
        L = (L & 7) * per + (L >> 3)
    bh = L // n_qtiles
    return bh, n_qtiles - 1 - (L - bh * n_qtiles)


SHAPES = list(itertools.product((1, 2, 3, 4, 8), (1, 2, 5, 8, 16, 32), (1, 255, 256, 2048, 8192, 9000)))


@pytest.mark.parametrize("causal", (False, True))
def test_block_order_is_a_bijection(causal):
    for B, H, N in SHAPES:
        tiles, grid, remap = plan_remap(B, H, N, causal)
        seen = {block_to_work(L, grid, B, H, tiles, remap) for L in range(grid)}
        assert len(seen) == grid, (B, H, N, causal)
        assert all(0 <= bh < B * H and 0 <= qt < tiles for bh, qt in seen)


def test_tile_major_order_for_short_causal_calls():
    # B=4, H=16, N=2048 (8 query tiles per head): each XCD starts with the
    # longest tile of each of its 8 heads
    tiles, grid, remap = plan_remap(4, 16, 2048, True)
    assert remap == 2
    first = [block_to_work(L, grid, 4, 16, tiles, remap) for L in range(64)]
    assert {qt for _, qt in first} == {tiles - 1}
    assert {bh for bh, _ in first} == set(range(64))
    # long sequences and non-causal calls keep the head-major order
    assert plan_remap(2, 16, 8192, True)[2] == 1
    assert plan_remap(4, 16, 2048, False)[2] == 1
