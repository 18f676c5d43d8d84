"""CPU model of how the GEMM kernels hand work items to workgroups.

A launch is sized from the padded row count (the host does not know the number
of valid rows); the kernels learn it on the device and map workgroup b to an
item XCD by XCD: the first pad8(real) workgroups cover the `real` items, each
XCD (b % 8) taking a contiguous range of them.  These tests check, for the
grid sizes the host code uses, that every item is computed exactly once --
including the forward's single-range case with more than 2048 token tiles,
whose grid once fell short of the padded item count and skipped items."""
import pytest


def pad8(n):
    return (n + 7) // 8 * 8


def xcd_item(b, nblocks):
    return (b % 8) * (nblocks // 8) + b // 8


def live_item(b, real):
    real8 = pad8(real)
    if b >= real8:
        return -1
    item = xcd_item(b, real8)
    return item if item < real else -1


def covered(grid, real):
    items = [live_item(b, real) for b in range(grid)]
    got = sorted(i for i in items if i >= 0)
    return got == list(range(real))


def fwd_grid(TT):
    # host: fwd_items = max(2048, TT); the launch covers pad8(fwd_items)
    return pad8(max(2048, TT))


@pytest.mark.parametrize("TT", [1, 7, 26, 2047, 2048, 2049, 2051, 2053, 3907, 65536])
def test_forward_items_single_range(TT):
    # P = 1: one vocabulary range per token tile, TTn = TT when every row is valid
    assert covered(fwd_grid(TT), TT)


@pytest.mark.parametrize("TT,P", [(26, 9), (26, 78), (100, 20), (2051, 1), (3907, 1)])
def test_forward_items_split(TT, P):
    # the device picks P with P * TTn <= max(2048, TT)
    assert P * TT <= max(2048, TT)
    assert covered(fwd_grid(TT), P * TT)


def test_short_grid_misses_items():
    # the grid of fwd_items workgroups (not rounded up) leaves items out when
    # the item count is not a multiple of 8: the case the rounding fixes
    assert not covered(2051, 2051)
    assert not covered(3907, 3907)


@pytest.mark.parametrize("TT,TTn", [(26, 26), (26, 13), (32, 1), (2051, 2049)])
@pytest.mark.parametrize("tiles_per_row", [1, 14, 64])
def test_backward_items(TT, TTn, tiles_per_row):
    # G / dX / dW tiles: grid pad8(kinds x TT) sized for the bound, real items
    # over the valid rows' TTn token tiles
    assert covered(pad8(tiles_per_row * TT), tiles_per_row * TTn)


def dx_parts_for(hidden_tiles, token_tiles, target, part_tiles):
    # the vocabulary parts of a launch's dX tiles (flce_kernels.h)
    if token_tiles <= 0:
        return 1
    per = hidden_tiles * token_tiles
    s = min(-(-target // per), 8)
    if part_tiles >= 0:
        s = min(s, 1 + part_tiles // token_tiles)
    return max(s, 1)


@pytest.mark.parametrize("H,C", [(3584, 6912), (4096, 6912), (2048, 6912), (1024, 3840),
                                 (3584, 3328), (2048, 3328), (1024, 1792),
                                 (256, 256), (2048, 1024), (65536, 256), (4096, 65536)])
def test_chunked_dx_grid_covers_every_chunk(H, C):
    # chunked mode: the part count is set per chunk on the device from the
    # chunk's rows; the host sizes the dX workgroups for the largest count any
    # chunk of at most C rows can take, and the part buffer for the extra parts
    HT, TTc, target = -(-H // 256), C // 256, 176
    full = dx_parts_for(HT, TTc, target, -1)
    part_tiles = max((full - 1) * TTc, min(-(-TTc // 2), 16))
    blocks = pad8(max(dx_parts_for(HT, tt, target, part_tiles) * HT * tt
                      for tt in range(1, TTc + 1)))
    assert dx_parts_for(HT, TTc, target, part_tiles) == full   # full chunks unchanged
    for tt in range(1, TTc + 1):
        s = dx_parts_for(HT, tt, target, part_tiles)
        assert (s - 1) * tt <= part_tiles                      # the parts fit the buffer
        assert covered(blocks, s * HT * tt)


def swz(row, chunk):
    # LDS byte offset of 16-byte chunk `chunk` of tile row `row` in a K-contiguous
    # slab (128-byte rows, flce_tile.h)
    return row * 128 + ((chunk ^ (row & 7) ^ ((row >> 3) & 1)) << 4)


def test_direct_to_lds_prefetch_fills_the_loaders_layout():
    # prefetch_direct: wave w, instruction j writes 1 KiB at the slab's row
    # 64 w + 8 j; lane l lands at 16 l past it and must fetch the (row, chunk)
    # that the register loader's commit stores at that address
    seen = {}
    for w in range(4):
        for j in range(8):
            row0 = 64 * w + 8 * j
            for lane in range(64):
                row = row0 + lane // 8
                chunk = (lane & 7) ^ (row & 7) ^ ((row >> 3) & 1)
                addr = row0 * 128 + 16 * lane
                assert swz(row, chunk) == addr
                assert (row, chunk) not in seen
                seen[(row, chunk)] = addr
    assert len(seen) == 256 * 8                       # every chunk of the slab once
    assert sorted(seen.values()) == list(range(0, 256 * 128, 16))
