"""CPU checks of the NT and MN-major kernels' tile orders (no GPU).

The persistent grid walks work units t = blockIdx.x, blockIdx.x + gridDim.x, ...
and maps each unit to an output tile.  The maps are restated here from the
kernel and the host set-up, and checked to be a bijection onto the tiles for
many shapes and grids: a tile that two units share is computed twice, one
that no unit reaches is never written.
"""
import numpy as np
import pytest

BAND_DENSE, BAND_CONTIGUOUS = 4, 8


def contiguous_params(tiles_m, tiles_n, grid):
    """Host side: the XCD-block part of the contiguous order."""
    blk = units = m0 = 0
    if grid % 8 == 0 and tiles_n % 2 == 0 and (grid // 8) % (tiles_n // 2) == 0:
        blk = (grid // 8) // (tiles_n // 2)
        rounds = tiles_m // (4 * blk)
        units, m0 = rounds * grid, rounds * 4 * blk
    band = BAND_CONTIGUOUS if tiles_m > BAND_CONTIGUOUS else tiles_m
    return blk, units, m0, band


def contiguous_tile(local, tiles_m, tiles_n, grid, params):
    blk, units, m0, band = params
    if local < units:
        sb, u = divmod(local, grid)
        x, j = u & 7, u >> 3
        return (sb * 4 + (x & 3)) * blk + j % blk, (x >> 2) * (tiles_n >> 1) + j // blk
    rest = local - units
    band_tiles = band * tiles_n
    b, in_band = divmod(rest, band_tiles)
    first_m = m0 + b * band
    rows = min(tiles_m - first_m, band)
    return first_m + in_band % rows, in_band // rows


def dense_tile(t, tiles_m, tiles_n, splits):
    num = tiles_m * tiles_n * splits
    per, extra = num >> 3, num & 7
    x = t & 7
    local = x * per + min(x, extra) + (t >> 3)
    split, local = local % splits, local // splits
    band = BAND_DENSE if tiles_m > BAND_DENSE else tiles_m
    b, in_band = divmod(local, band * tiles_n)
    first_m = b * band
    rows = min(tiles_m - first_m, band)
    return first_m + in_band % rows, in_band // rows, split


CONTIGUOUS_CASES = [(200, 16, 256), (18, 16, 256), (16, 16, 256), (15, 16, 256), (7, 16, 256),
                    (130, 2, 256), (64, 4, 256), (9, 32, 256), (40, 64, 256), (33, 6, 256),
                    (20, 16, 128), (20, 16, 136), (3, 1, 3), (50, 8, 64), (1, 1, 2)]


@pytest.mark.parametrize("tiles_m,tiles_n,grid", CONTIGUOUS_CASES)
def test_contiguous_order_is_a_bijection(tiles_m, tiles_n, grid):
    params = contiguous_params(tiles_m, tiles_n, grid)
    per_group = tiles_m * tiles_n
    for half in range(2):   # each tile is listed twice, once per 128-row block
        got = [contiguous_tile(t - half * per_group, tiles_m, tiles_n, grid, params)
               for t in range(half * per_group, (half + 1) * per_group)]
        assert sorted(got) == [(m, n) for m in range(tiles_m) for n in range(tiles_n)]


def test_contiguous_xcd_blocks_are_compact():
    """At 256 workgroups and 16 N tiles, the 32 tiles an XCD holds in one round
    of the grid span 4 M tiles x 8 N tiles, and one round covers 16 x 16."""
    tiles_m, tiles_n, grid = 200, 16, 256
    params = contiguous_params(tiles_m, tiles_n, grid)
    assert params[:3] == (4, 12 * 256, 192)
    for rnd in range(12):
        tiles = [contiguous_tile(rnd * grid + u, tiles_m, tiles_n, grid, params) for u in range(grid)]
        assert {m for m, _ in tiles} == set(range(16 * rnd, 16 * rnd + 16))
        for x in range(8):
            mine = tiles[x::8]
            assert len({m for m, _ in mine}) == 4 and len({n for _, n in mine}) == 8


@pytest.mark.parametrize("tiles_m,tiles_n,splits", [(16, 9, 1), (1, 4, 8), (5, 3, 2), (57, 28, 1), (2, 2, 3)])
def test_dense_order_is_a_bijection(tiles_m, tiles_n, splits):
    num = tiles_m * tiles_n * splits
    got = sorted(dense_tile(t, tiles_m, tiles_n, splits) for t in range(num))
    assert got == [(m, n, s) for m in range(tiles_m) for n in range(tiles_n) for s in range(splits)]


def tn_xcd_blocks(tiles_m, tiles_n):
    """Host side of the MN-major kernel's order: 8 equal blocks whose sides
    divide the grid, fewest panels (block height + width) first."""
    best, blk = None, (0, 0)
    if (tiles_m * tiles_n) % 8:
        return blk
    for bxm in (1, 2, 4, 8):
        bxn = 8 // bxm
        if tiles_m % bxm or tiles_n % bxn:
            continue
        cost = tiles_m // bxm + tiles_n // bxn
        if best is None or cost < best:
            best, blk = cost, (tiles_m // bxm, tiles_n // bxn)
    return blk


def tn_tile(local, tiles_m, tiles_n, blk):
    tm, tn = local % tiles_m, local // tiles_m
    bm, bn = blk
    if bm:
        x, j = local & 7, local >> 3
        bxm = tiles_m // bm
        tm, tn = (x % bxm) * bm + j % bm, (x // bxm) * bn + j // bm
    return tm, tn


@pytest.mark.parametrize("tiles_m,tiles_n", [(8, 16), (16, 16), (1, 8), (2, 4), (8, 1), (3, 8), (12, 16),
                                             (5, 8), (16, 2), (7, 7), (1, 1), (6, 4), (32, 64)])
def test_tn_order_is_a_bijection(tiles_m, tiles_n):
    blk = tn_xcd_blocks(tiles_m, tiles_n)
    got = sorted(tn_tile(l, tiles_m, tiles_n, blk) for l in range(tiles_m * tiles_n))
    assert got == [(m, n) for m in range(tiles_m) for n in range(tiles_n)]


def test_tn_xcd_blocks_are_compact():
    """K-grouped MoE weight gradient (M = 2048, N = 4096: 8 x 16 tiles per
    group): each XCD takes a 4 x 4 block of every group, so its tiles share 4 A
    and 4 B panels instead of 1 A panel and all 16 B panels."""
    tiles_m, tiles_n = 8, 16
    blk = tn_xcd_blocks(tiles_m, tiles_n)
    assert blk == (4, 4)
    for x in range(8):
        mine = [tn_tile(l, tiles_m, tiles_n, blk) for l in range(x, tiles_m * tiles_n, 8)]
        assert len({m for m, _ in mine}) == 4 and len({n for _, n in mine}) == 4
    assert tn_xcd_blocks(16, 16) == (8, 4)     # 4096 x 4096 dense layouts: 12 panels per XCD
    assert tn_xcd_blocks(7, 7) == (0, 0)       # 49 tiles do not split into 8 blocks
