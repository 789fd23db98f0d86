"""Work order and mask segments of the attention kernels, as a Python model.

These tests check a Python restatement of the device and host logic, not the
compiled code: plan_remap / plan_persist / block_to_work / item_of below
re-implement plan() (attn_api.cpp), block_to_work and item_of
(attn_kernels.hpp), and the segment bounds
re-implement the kernels' loop limits.  They pin the design -- that the
chosen orders are bijections and that the segment bounds agree with the
per-tile mask definition -- so a change to the model that breaks it fails
here.  Whether the compiled kernels follow the model is checked on the GPU:
every parity test covers each query tile's rows (sampled or whole) and the
guard bands around O and LSE, so a launch index mapped twice or never shows
there as a wrong or missing row.

Block order: the fixed-length forward kernels must map every item index to
a distinct (batch*head, query tile) pair, so that each query tile is
computed exactly once; in a persistent launch every item must be taken by
exactly one work-group, on its own XCD, and a causal call's work must
spread evenly over the work-groups.

Mask segments: the forward, dQ and dK/dV tile loops run the tiles that need
no mask through a body without it; the segment bounds must agree with the
per-tile definition of a masked tile."""

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


def plan_persist(grid, remap, cus):
    """plan(): one work-group per compute unit when the block order is
    XCD-aware (fixed-length calls) and there are more items than units."""
    return remap != 0 and cus >= 8 and cus % 8 == 0 and grid > cus


def item_of(g, s, G, items):
    """item_of (attn_kernels.hpp): item of persistent work-group g at step s,
    or None past its XCD's last item."""
    j, W = g >> 3, G >> 3
    k = s * W + (W - 1 - j if s & 1 else j)
    if k >= items >> 3:
        return None
    return (g & 7) + 8 * k


def persistent_schedule(grid, cus):
    """Items of each work-group, in its order."""
    out = []
    for g in range(cus):
        mine, s = [], 0
        while True:
            L = item_of(g, s, cus, grid)
            if L is None:
                break
            mine.append(L)
            s += 1
        out.append(mine)
    return out


@pytest.mark.parametrize("cus", (256, 64, 8))
def test_persistent_order_covers_every_item_once(cus):
    for B, H, N in SHAPES:
        for causal in (False, True):
            tiles, grid, remap = plan_remap(B, H, N, causal)
            if not plan_persist(grid, remap, cus):
                continue
            sched = persistent_schedule(grid, cus)
            flat = [L for mine in sched for L in mine]
            assert sorted(flat) == list(range(grid)), (B, H, N, causal, cus)
            # a work-group stays on its XCD's items
            assert all(L % 8 == g % 8 for g, mine in enumerate(sched) for L in mine)


@pytest.mark.parametrize("B,H,N", [(2, 16, 8192), (1, 32, 32768), (4, 16, 2048), (2, 32, 8192)])
def test_persistent_order_balances_causal_work(B, H, N):
    # work of an item: the 64-key tiles its 256 query rows see (causal)
    tiles, grid, remap = plan_remap(B, H, N, True)
    assert plan_persist(grid, remap, 256)
    sched = persistent_schedule(grid, 256)
    work = [sum((block_to_work(L, grid, B, H, tiles, remap)[1] + 1) * 4 for L in mine)
            for mine in sched]
    assert max(work) <= 1.03 * (sum(work) / len(work)), (B, H, N, max(work), min(work))


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


# ---------------------------------------------------------------------------
# Mask segments.  The kernels run the tiles that need no mask through a body
# without it; the bounds below restate the kernels' formulas and are checked
# against the per-tile definition of "needs the mask".
# ---------------------------------------------------------------------------

def _fwd_first_masked(N, BC, causal, qw0):
    # attn_fwd_bf16.hip / attn_fwd_fp8.hip and the dQ kernel: first key tile
    # of a wave (32 queries from qw0) that needs the mask
    fm = N // BC
    if causal:
        fm = min(fm, (qw0 + 1) // BC)
    return fm


def _fwd_tile_masked(N, BC, causal, qw0, t):
    kv0 = t * BC
    return (kv0 + BC > N) or (causal and kv0 + BC - 1 > qw0)


@pytest.mark.parametrize("BC", (64, 128))
def test_forward_mask_segments(BC):
    for N in list(range(1, 1200, 7)) + [2048, 8191, 8192, 8193]:
        n_kv = -(-N // BC)
        for causal in (False, True):
            for qw0 in range(0, N, 32):
                T = min(qw0 + 31, N - 1) // BC + 1 if causal else n_kv
                fm = _fwd_first_masked(N, BC, causal, qw0)
                for t in range(T):
                    assert (t >= fm) == _fwd_tile_masked(N, BC, causal, qw0, t), (N, causal, qw0, t)


def test_backward_dkdv_mask_segments():
    # attn_bwd_bf16.hip, dK/dV kernel: 256 keys per work-group, 32 per wave,
    # 64-query tiles; segments inactive / masked / unmasked / masked
    BQ, BK = 64, 256
    for N in list(range(1, 1500, 11)) + [2048, 8191, 8192, 8193]:
        n = -(-N // BQ)
        for causal in (False, True):
            for kt in range(-(-N // BK)):
                k0 = kt * BK
                first = k0 // BQ if causal else 0
                for wave in range(8):
                    kw0 = k0 + wave * 32
                    j_act = n if kw0 >= N else (max(first, kw0 // BQ) if causal else first)
                    j_um = max(j_act, (kw0 + 31 + BQ - 1) // BQ) if causal else j_act
                    seg_b = max(j_act, min(j_um, n))
                    seg_c = max(seg_b, min(N // BQ, n))
                    for j in range(first, n):
                        qt0 = j * BQ
                        active = kw0 < N and ((not causal) or qt0 + BQ - 1 >= kw0)
                        masked = (qt0 + BQ > N) or (causal and qt0 < kw0 + 31)
                        if j < min(j_act, n):
                            got = None
                        else:
                            got = not (seg_b <= j < seg_c)
                        assert got == (masked if active else None), (N, causal, kt, wave, j)
