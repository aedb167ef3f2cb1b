"""The B = 32 tile numbering of the decode kernel, modelled on the host (no GPU).

At B = 32 the decode's plain runs give the two 16-token tiles of a block
whose tokens span both halves (32 blk + 16 < L) alternate groups of four
tokens: row r of the block's first tile is token 8 (r / 4) + r % 4, of its
second that + 4.  A last block of at most 16 tokens stays one tile in token
order.  Lane group g holds rows 4g .. 4g + 3 of a tile; its V values for
both tiles of a paired block are one 16-byte piece of each dim row (tokens
8g .. 8g + 7).

This module restates those formulas in Python and checks what the kernel
relies on, for every length up to a few blocks:

* the tiles 0 .. ceil(L / 16) - 1 hold every token of [0, L) exactly once,
  and no other token below the block's end (the rest are masked as >= L);
* a lane group's tokens in the two tiles of a paired block are the 8
  consecutive tokens of one 16-byte piece of a V dim row, first tile low half;
* the appended token L - 1 is row rt_new of tile tile_new, and the row the
  write-back stores for that row is the token's own K row and V position;
* the per-lane K byte offset of a paired tile's row, plus the half's shift,
  is that token's row in the block.
"""

import pytest

TILE = 16
B = 32


def tile_rows(t, L):
    """Block tokens of tile t's rows 0..15 (the kernel's numbering)."""
    blk0 = (t * TILE) // B * B
    half = t % 2
    if blk0 + TILE < L:  # paired block
        return [blk0 + 8 * (r // 4) + r % 4 + 4 * half for r in range(TILE)]
    return [t * TILE + r for r in range(TILE)]


def lane_first_token(t, grp, L):
    """The consume loop's `first`: token of element 0 of lane group grp."""
    t0 = t * TILE
    blk0 = t0 & ~(B - 1)
    if blk0 + TILE < L:
        return blk0 + 8 * grp + 4 * ((t0 // TILE) & 1)
    return t0 + 4 * grp


def new_row(L):
    """tile_new, rt_new of the run set-up for the appended token L - 1."""
    tile_new = (L + TILE - 1) // TILE - 1
    rt_new = L - 1 - tile_new * TILE
    blk0 = (L - 1) & ~(B - 1)
    off = L - 1 - blk0
    if blk0 + TILE < L:
        tile_new = blk0 // TILE + ((off >> 2) & 1)
        rt_new = 4 * (off >> 3) + (off & 3)
    return tile_new, rt_new


@pytest.mark.parametrize("L", range(1, 5 * B + 1))
def test_tiles_cover_each_token_once(L):
    ntile = (L + TILE - 1) // TILE
    seen = []
    for t in range(ntile):
        rows = tile_rows(t, L)
        # every row is a token of the tile's block; tokens past L are masked
        blk0 = (t * TILE) // B * B
        assert all(blk0 <= x < blk0 + B for x in rows)
        seen += [x for x in rows if x < L]
        # the lanes' first tokens agree with the rows they hold
        for g in range(4):
            first = lane_first_token(t, g, L)
            assert [first + i for i in range(4)] == rows[4 * g:4 * g + 4]
    assert sorted(seen) == list(range(L))


@pytest.mark.parametrize("L", range(1, 5 * B + 1))
def test_lane_group_v_piece(L):
    """One 16-byte load (8 tokens) per lane group feeds both tiles of a pair."""
    for blk in range((L + B - 1) // B):
        blk0 = blk * B
        if not blk0 + TILE < L:
            continue
        t = blk0 // TILE
        for g in range(4):
            first_a = lane_first_token(t, g, L)
            first_b = lane_first_token(t + 1, g, L)
            # byte offsets in the 64-byte dim row: 16 g for the piece
            assert 2 * (first_a - blk0) == 16 * g
            assert first_b == first_a + 4  # the piece's upper 8 bytes


@pytest.mark.parametrize("L", range(1, 5 * B + 1))
def test_appended_row_position(L):
    tile_new, rt_new = new_row(L)
    assert 0 <= tile_new < (L + TILE - 1) // TILE
    assert tile_rows(tile_new, L)[rt_new] == L - 1
    # write-back: K row of row rt (k_off's row rt plus the half's shift) and
    # V at 8 g + (8 g + 8 half) bytes into the dim row, g = rt / 4
    blk0 = (L - 1) & ~(B - 1)
    half = tile_new % 2
    if blk0 + TILE < L:
        k_row = rt_new + (8 * (rt_new // 4) + rt_new % 4 + 4 * half - rt_new)
        assert blk0 + k_row == L - 1
        g = rt_new // 4
        v_byte = 8 * g + (8 * g + 8 * half) + 2 * (rt_new % 4)
        assert v_byte == 2 * (L - 1 - blk0)
    else:
        assert tile_new * TILE + rt_new == L - 1


def test_paired_k_offsets():
    """k_off_pair (row 8 (col / 4) + col % 4) plus 4 rows for the second
    tile is the block row of that tile's row col."""
    L = 2 * B
    for half in (0, 1):
        rows = tile_rows(half, L)
        for col in range(TILE):
            assert 8 * (col // 4) + col % 4 + 4 * half == rows[col]
